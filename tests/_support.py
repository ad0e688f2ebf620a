"""Shared helpers of the GPU parity tests: run the HIP library through the C
ABI, run the CPU oracle on the same seeded inputs, compare to the bars the
tests state (routing bit-exact up to near-ties, dispatch bit-exact, outputs
within the fp32 / bf16 tolerances)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparsely_gated_mixture_amd as moe
from sparsely_gated_mixture_amd.workloads import (DTYPE_BF16, DTYPE_F32, DTYPE_FP8, make_inputs,
                                                  to_numpy64)

TOL_F32 = 1e-4     # max-abs-normalised, fp32 experts
TOL_BF16 = 2e-2    # max-abs-normalised, bf16 experts
TOL_AUX = 1e-4     # relative, aux losses (1e-7 absolute floor)
# Gate weights: the fp32 bar of the layer (1e-4 relative) with a 1e-6 floor.
# The logits come from fp32 dot products over d = 512..7168 terms, whose
# rounding (measured up to 2.6e-6 absolute, 1.1e-5 relative on the weights)
# is above a pure 1e-6 absolute bar.
TOL_W_REL = 1e-4
TOL_W = 1e-6
NEAR_TIE = 1e-4    # relative gap of adjacent sorted H that counts as a tie
MISMATCH_BUDGET = 1e-4  # fraction of tokens allowed to route differently


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_inputs(cfg, T=None):
    torch.cuda.synchronize()
    return make_inputs(cfg, device="cuda", T=T)


def host(inp, keys=None):
    keys = keys or [k for k in inp if k not in ("w1", "w3", "w2", "b1", "b2")]
    return {k: to_numpy64(inp[k]) for k in keys}


def expert_weights_host(inp, experts):
    """float64 host copies of the listed experts' weights."""
    out = {}
    for name in ("w1", "w3", "w2", "b1", "b2"):
        t = inp.get(name)
        out[name] = None if t is None else {int(e): to_numpy64(t[int(e)]) for e in experts}
    return out


def gpu_forward(cfg, inp, stream=None):
    """Whole layer through moe_forward; returns host copies of y, losses and
    every intermediate."""
    T, k, n = inp["x"].shape[0], cfg.k, cfg.n_experts
    c = cfg.replace(T=T)
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    diag = dict(topk_idx=torch.empty((T, k), **i32), topk_w=torch.empty((T, k), **f32),
                importance=torch.empty(n, **f32), load=torch.zeros(n, **f32),
                counts_pre=torch.empty(n, **i32), counts=torch.empty(n, **i32),
                offsets=torch.empty(n + 1, **i32), perm=torch.full((max(T * k, 1),), -7, **i32),
                slot_pos=torch.empty((T, k), **i32))
    layer = moe.MoELayer(c, inp)
    y, losses = layer.forward(inp["x"], inp.get("noise"), inp.get("noise2"), diag=diag)
    torch.cuda.synchronize()
    out = {kk: v.cpu().numpy() for kk, v in diag.items()}
    out["y"] = y.cpu().double().numpy()
    out["losses"] = losses.cpu().double().numpy()
    return out


def sorted_gaps_near_tie(H_row, k):
    """True if any adjacent pair among the top-(k+1) values of H_row is
    within NEAR_TIE relative distance (a tie the fp32 gate may order
    differently from the float64 oracle)."""
    v = np.sort(H_row)[::-1][:min(k + 1, len(H_row))]
    for a, b in zip(v[:-1], v[1:]):
        if a - b < NEAR_TIE * max(abs(a), abs(b)):
            return True
    return False


def routing_mismatches(gpu_idx, orc_idx, H, k, budget=MISMATCH_BUDGET):
    """Tokens whose slots differ; asserts each is a near-tie, that every slot
    the GPU chose holds a value within the near-tie distance of the oracle's
    value of that rank (so the GPU's selection is a valid top-k), and that
    their count is within the budget.  Returns the mismatching token ids."""
    bad = np.nonzero(np.any(gpu_idx != orc_idx, axis=1))[0]
    T = gpu_idx.shape[0]
    for t in bad:
        assert sorted_gaps_near_tie(H[t], k), (
            f"token {t} routes differently without a near-tie: gpu {gpu_idx[t]} "
            f"oracle {orc_idx[t]}")
        ranked = np.sort(H[t])[::-1][:k]
        chosen = H[t][gpu_idx[t]]
        assert len(set(gpu_idx[t].tolist())) == k, f"token {t}: repeated expert"
        assert np.all(np.abs(chosen - ranked) <=
                      NEAR_TIE * np.maximum(np.abs(chosen), np.abs(ranked))), (
            f"token {t}: the GPU's slots {gpu_idx[t]} are not a top-{k} within the near-tie "
            f"distance")
    assert len(bad) <= budget * T, f"{len(bad)} near-tie mismatches of {T} tokens"
    if len(bad):
        log(f"  near-tie routing mismatches: {len(bad)} of {T}")
    return bad


def max_abs_norm(a, ref):
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return float(np.max(np.abs(a - ref)) / scale)


def assert_close_rel(a, b, rel, floor=1e-7, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b)
    lim = rel * np.abs(b) + floor
    assert np.all(err <= lim), f"{what}: max err {err.max()} vs limit {lim[np.argmax(err - lim)]}"


def check_dispatch_exact(cfg, gpu, T):
    """Dispatch is bit-exact against the oracle's dispatch of the GPU's own
    routing."""
    d = oracle.dispatch(gpu["topk_idx"], cfg.n_experts, cfg.capacity_factor)
    np.testing.assert_array_equal(gpu["counts_pre"], d["counts_pre"])
    np.testing.assert_array_equal(gpu["counts"], d["counts"])
    np.testing.assert_array_equal(gpu["offsets"], d["offsets"])
    rows = d["rows"]
    np.testing.assert_array_equal(gpu["perm"][:rows], d["perm"])
    np.testing.assert_array_equal(gpu["slot_pos"], d["slot_pos"])
    return d


def fp8_dequant(w):
    """The values FP8 experts compute with: the oracle's E4M3 row
    quantization of the bf16 weights, dequantized."""
    return oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(w))


def fp8_view(ew):
    """expert_weights_host dict with every w1/w3/w2 matrix dequantized."""
    out = dict(ew)
    for name in ("w1", "w3", "w2"):
        if ew.get(name) is not None:
            out[name] = {e: fp8_dequant(m) for e, m in ew[name].items()}
    return out


def oracle_flat(cfg, h, ew):
    if cfg.expert_dtype == DTYPE_FP8:
        ew = fp8_view(ew)
    return oracle.forward(
        h["x"], h["w_gate"], cfg.k, _stack(ew["w1"]), _stack(ew["w2"]), b_gate=h.get("b_gate"),
        w_noise=h.get("w_noise"), noise=h.get("noise"), b1=_stack(ew["b1"]), w3=_stack(ew["w3"]),
        b2=_stack(ew["b2"]), mode=cfg.gate, act=cfg.act, bf16=cfg.expert_dtype != DTYPE_F32,
        capacity_factor=cfg.capacity_factor, w_importance=cfg.w_importance, w_load=cfg.w_load,
        alpha=cfg.alpha_switch, w_z=cfg.w_z, w_entropy=cfg.w_entropy, ws1=h.get("ws1"),
        ws3=h.get("ws3"), ws2=h.get("ws2"))


def _stack(dct):
    if dct is None:
        return None
    return np.stack([dct[e] for e in sorted(dct)])


def y_tolerance(cfg):
    return TOL_F32 if cfg.expert_dtype == DTYPE_F32 else TOL_BF16


def oracle_gate_any(cfg, h):
    """Oracle gating of a flat or two-level config on host inputs `h`.
    Returns (topk_idx, topk_w, importance, load, H_for_ties, near_tie, zsum,
    entsum)."""
    if cfg.hierarchical:
        gh = oracle.gate_hier(h["x"], h["w_gate"], h.get("w_noise"), h.get("noise"),
                              cfg.k_groups, h["w_gate2"], h.get("w_noise2"), h.get("noise2"),
                              cfg.k2, b_gate=h.get("b_gate"))
        return (gh["topk_idx"], gh["topk_w"], gh["importance"], gh["load"], None,
                gh["near_tie"], gh["zsum"], gh["entsum"])
    g = oracle.gate(h["x"], h["w_gate"], cfg.k, h.get("b_gate"), h.get("w_noise"),
                    h.get("noise"), cfg.gate)
    return g.topk_idx, g.topk_w, g.importance, g.load, g.H, g.near_tie, g.zsum, g.entsum


def check_routing_any(cfg, gpu_idx, orc_idx, H, near_tie):
    """Routing check for flat (sorted-gap rule on H) or two-level configs
    (the oracle's per-level near-tie flags)."""
    if H is not None:
        return routing_mismatches(gpu_idx, orc_idx, H, cfg.k)
    bad = np.nonzero(np.any(gpu_idx != orc_idx, axis=1))[0]
    for t in bad:
        assert near_tie[t], f"token {t} routes differently without a near-tie"
    assert len(bad) <= MISMATCH_BUDGET * gpu_idx.shape[0]
    return bad


def expert_weights_f64(cfg, inp, e):
    """float64 host copies of expert e's weights (converted on the device,
    one expert at a time); FP8 experts as the values their codes stand for."""
    out = {}
    for name in ("w1", "w3", "w2", "b1", "b2"):
        t = inp.get(name)
        if t is None:
            out[name] = None
            continue
        m = t[e].to(torch.float64).cpu().numpy()
        if cfg.expert_dtype == DTYPE_FP8 and name in ("w1", "w3", "w2"):
            m = fp8_dequant(m)
        out[name] = m
    return out


def expert_rows_reference(cfg, inp, x64, perm, offsets, rows_by_expert):
    """The oracle's expert output rows y_perm[r] for the requested rows of
    each expert (rows_by_expert: expert -> global rows of the merged batch),
    computed expert by expert from the device's weights."""
    bf = cfg.expert_dtype != DTYPE_F32
    out = {}
    for e in sorted(rows_by_expert):
        rows = np.asarray(sorted(rows_by_expert[e]), np.int64)
        if len(rows) == 0:
            continue
        assert np.all((rows >= offsets[e]) & (rows < offsets[e + 1]))
        w = expert_weights_f64(cfg, inp, e)
        ys = oracle.expert_ffn(x64[perm[rows]], w["w1"], w["w2"], b1=w["b1"], w3=w["w3"],
                               b2=w["b2"], act=cfg.act, bf16=bf)
        for r, v in zip(rows, ys):
            out[int(r)] = v
    return out


def shared_reference(cfg, inp, x64, tokens):
    """The shared expert's output on `tokens` (zeros without one)."""
    if not cfg.d_hidden_shared:
        return np.zeros((len(tokens), cfg.d_model))
    ws = {k: (None if inp.get(k) is None else inp[k].to(torch.float64).cpu().numpy())
          for k in ("ws1", "ws3", "ws2")}
    return oracle.expert_ffn(x64[tokens], ws["ws1"], ws["ws2"], w3=ws["ws3"], act=cfg.act,
                             bf16=cfg.expert_dtype != DTYPE_F32)


def covering_tokens(gpu, disp, T, n_random=16, seed=0):
    """Tokens whose outputs, checked together, exercise every non-empty
    expert: the ends of the batch; the rows of the hottest expert's last
    128-row tile (its first, second and last rows); every single-row expert;
    then, experts in ascending order of rows, the token of one row of each
    expert not yet covered; plus a few random tokens."""
    counts, offsets, perm = disp["counts"], disp["offsets"], disp["perm"]
    idx, slot_pos = gpu["topk_idx"], gpu["slot_pos"]
    r = np.random.default_rng(seed)
    chosen = [0, 1, T - 2, T - 1] if T >= 4 else list(range(T))
    hot = int(np.argmax(counts))
    lo, hi = int(offsets[hot]), int(offsets[hot + 1])
    tile0 = lo + (hi - lo - 1) // 128 * 128
    chosen += [int(perm[q]) for q in (tile0, min(tile0 + 1, hi - 1), hi - 2, hi - 1) if q >= lo]
    chosen += [int(perm[offsets[e]]) for e in np.nonzero(counts == 1)[0]]
    covered = set()

    def cover(t):
        covered.update(int(e) for e, p in zip(idx[t], slot_pos[t]) if p >= 0)
    for t in chosen:
        cover(t)
    for e in np.argsort(counts, kind="stable"):
        if counts[e] == 0 or int(e) in covered:
            continue
        q = int(offsets[e]) + int(r.integers(counts[e]))
        chosen.append(int(perm[q]))
        cover(int(perm[q]))
    chosen += [int(t) for t in r.choice(T, size=min(T, n_random), replace=False)]
    assert covered >= {int(e) for e in np.nonzero(counts)[0]}
    return np.unique(np.asarray(chosen, np.int64))


def oracle_gate_on_routing(cfg, h, idx):
    """The oracle's Importance, Load and losses with the gate's selection
    held at `idx` (the GPU's routing): the weights and load terms come from
    the oracle's own logits, so tokens that route differently at a near-tie
    count the way the GPU routed them instead of being left out."""
    T, k, n = idx.shape[0], cfg.k, cfg.n_experts
    if cfg.hierarchical:
        gh = oracle.gate_hier(h["x"], h["w_gate"], h.get("w_noise"), h.get("noise"),
                              cfg.k_groups, h["w_gate2"], h.get("w_noise2"), h.get("noise2"),
                              cfg.k2, b_gate=h.get("b_gate"), route=idx)
        imp, ld, zsum, entsum = gh["importance"], gh["load"], gh["zsum"], gh["entsum"]
    else:
        g = oracle.gate(h["x"], h["w_gate"], k, h.get("b_gate"), h.get("w_noise"),
                        h.get("noise"), cfg.gate, route=idx)
        imp, ld, zsum, entsum = g.importance, g.load, g.zsum, g.entsum
    counts_pre = oracle.dispatch(idx, n, cfg.capacity_factor)["counts_pre"]
    losses = oracle.aux(T, k, imp, ld, counts_pre, cfg.w_importance, cfg.w_load,
                        cfg.alpha_switch, zsum, entsum, cfg.w_z, cfg.w_entropy)
    return imp, ld, losses, zsum, entsum


def check_aux(cfg, h, gpu):
    imp, ld, losses, _, _ = oracle_gate_on_routing(cfg, h, gpu["topk_idx"])
    assert_close_rel(gpu["importance"], imp, 1e-5, 1e-5, "importance")
    if ld is not None:
        assert_close_rel(gpu["load"], ld, 1e-5, 1e-5, "load")
    assert_close_rel(gpu["losses"], losses, TOL_AUX, 1e-7, "losses")


def full_size_check(cfg, every_token=False, n_random=16, seed=0):
    """Full-size forward of `cfg` through moe_forward against the oracle:
    routing of every token (bit-exact up to near ties), gate weights,
    dispatch bit-exact, Importance / Load / losses (the oracle held at the
    GPU's routing), and y element-wise -- on every token, or on tokens that
    cover every non-empty expert (covering_tokens) -- from the oracle's
    experts evaluated expert by expert."""
    log(f"[full-size] {cfg.name} T={cfg.T} d={cfg.d_model} h={cfg.d_hidden} "
        f"n={cfg.n_experts} k={cfg.k}")
    inp = dev_inputs(cfg)
    gpu = gpu_forward(cfg, inp)
    h = host(inp)
    oidx, ow, oimp, oload, H, near, zsum, entsum = oracle_gate_any(cfg, h)
    bad = check_routing_any(cfg, gpu["topk_idx"], oidx, H, near)
    ok = np.setdiff1d(np.arange(cfg.T), bad)
    np.testing.assert_allclose(gpu["topk_w"][ok], ow[ok], rtol=TOL_W_REL, atol=TOL_W)
    d = check_dispatch_exact(cfg, gpu, cfg.T)
    check_aux(cfg, h, gpu)
    if every_token:
        tokens = ok
    else:
        tokens = np.intersect1d(covering_tokens(gpu, d, cfg.T, n_random, seed), ok)
    rows_by_expert = {}
    for t in tokens:
        for e, p in zip(gpu["topk_idx"][t], gpu["slot_pos"][t]):
            if p >= 0:
                rows_by_expert.setdefault(int(e), []).append(int(p))
    yp = expert_rows_reference(cfg, inp, h["x"], d["perm"], d["offsets"], rows_by_expert)
    ys = shared_reference(cfg, inp, h["x"], tokens)
    for i, t in enumerate(tokens):
        for s in range(cfg.k):
            p = gpu["slot_pos"][t, s]
            if p >= 0:
                ys[i] += ow[t, s] * yp[int(p)]
    err = max_abs_norm(gpu["y"][tokens], ys)
    experts = len(rows_by_expert)
    log(f"  routing mismatches {len(bad)}, kept rows {d['rows']}, checked tokens {len(tokens)} "
        f"covering {experts} of {int(np.count_nonzero(d['counts']))} non-empty experts, "
        f"y error {err:.3e}")
    assert experts == int(np.count_nonzero(d["counts"]))
    assert err <= y_tolerance(cfg)
    return gpu


def full_parity(cfg, T=None, aux=True, tie_budget=MISMATCH_BUDGET):
    """End-to-end forward of `cfg` (T tokens) against the oracle, element by
    element.  tie_budget: the fraction of tokens that may route differently
    at a near-tie (the workloads' bar is 0.01 %; edge-case layouts whose
    top-(k+1) values crowd together pass 1)."""
    T = cfg.T if T is None else T
    c = cfg.replace(T=T)
    log(f"[parity] {cfg.name} T={T} d={c.d_model} h={c.d_hidden} n={c.n_experts} k={c.k}")
    inp = dev_inputs(c, T)
    gpu = gpu_forward(c, inp)
    h = host(inp)
    ew = expert_weights_host(inp, range(c.n_experts))
    ref = oracle_flat(c, h, ew)
    g = ref["gate"]
    bad = routing_mismatches(gpu["topk_idx"], g.topk_idx, g.H, c.k, tie_budget)
    ok = np.setdiff1d(np.arange(T), bad)
    np.testing.assert_allclose(gpu["topk_w"][ok], g.topk_w[ok], rtol=TOL_W_REL, atol=TOL_W)
    d = check_dispatch_exact(c, gpu, T)
    if len(bad) == 0:
        np.testing.assert_array_equal(d["perm"], ref["dispatch"]["perm"])
    err = max_abs_norm(gpu["y"][ok], ref["y"][ok])
    log(f"  y max-abs-normalised error {err:.3e}")
    assert err <= y_tolerance(c)
    if aux and len(bad) == 0:
        assert_close_rel(gpu["importance"], g.importance, 1e-5, 1e-5, "importance")
        if g.load is not None:
            assert_close_rel(gpu["load"], g.load, 1e-5, 1e-5, "load")
        assert_close_rel(gpu["losses"], ref["losses"], TOL_AUX, 1e-7, "losses")
    elif aux:
        check_aux(c, h, gpu)
    return gpu, ref
