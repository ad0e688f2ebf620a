"""Parity of the backward pass (moe_backward through the C ABI) against the
oracle's backward on the same seeded inputs.

Bar: every gradient tensor within 2e-2 max-abs-normalised of the oracle's
for bf16 experts (the bf16 bar of the layer: the expert products round their
operands to bf16 -- the gradient rows entering them as well -- and
accumulate in fp32; the oracle computes in fp64 with the forward's
bf16-rounded inputs and hidden activations), 1e-4 for fp32 experts.  The discrete decisions must be the oracle's: the routing is
compared exactly, and for a noisy gate, whose load estimator sends part of a
token's gradient to the logit of the rank-k expert (the largest one not
kept), the cases use inputs where the k+1-th and k+2-th largest gate values
are not within 1e-4 of each other (checked).  ReLU'(0) is undefined: where
a pre-activation lies within rounding of zero (the oracle flags |pre| <= 2e-5
of the sum of its terms' magnitudes), the GPU's fp32 mask may take either
value; an entry that such a pre-activation feeds may differ from the
oracle's by at most the oracle's bound on that choice ("slack") plus the bar,
and every other entry meets the bar.
"""
import numpy as np
import pytest
import torch

import oracle
from _support import TOL_BF16, TOL_F32, log, max_abs_norm
from sparsely_gated_mixture_amd import MoELayer, moe_gate_k_splits
from sparsely_gated_mixture_amd.workloads import (ACT_SWIGLU, DTYPE_F32, GATE_SIGMOID_BIAS,
                                                  GATE_SWITCH_TOP1, PRESETS, MoEConfig,
                                                  make_grad_inputs, make_inputs, to_numpy64)

pytestmark = pytest.mark.gpu

CASES = {
    # noisy top-4 softmax, ReLU with biases, logit bias, capacity drops; 16 experts,
    # several 128-row tiles and ragged ones
    "lm_small": MoEConfig("bwd_lm_small", T=640, d_model=128, d_hidden=192, n_experts=16, k=4,
                          capacity_factor=1.0, logit_bias="normal0.5", expert_bias_std=0.1,
                          seed=2101),
    # Switch top-1 with capacity, noiseless, ReLU without biases
    "switch": MoEConfig("bwd_switch", T=512, d_model=128, d_hidden=256, n_experts=8, k=1,
                        gate=GATE_SWITCH_TOP1, noisy=False, capacity_factor=1.25,
                        logit_bias="normal1", seed=2102),
    # sigmoid gate with selection-only bias, SwiGLU experts, shared SwiGLU expert
    "sigmoid_shared": MoEConfig("bwd_sigmoid_shared", T=320, d_model=128, d_hidden=128,
                                n_experts=16, k=4, act=ACT_SWIGLU, gate=GATE_SIGMOID_BIAS,
                                noisy=False, logit_bias="normal0.5", d_hidden_shared=192,
                                seed=2103),
    # renormalised top-8 of 32 SwiGLU experts, Zipf logit bias (the fine-grained layer)
    "swiglu_top8": MoEConfig("bwd_swiglu_top8", T=256, d_model=192, d_hidden=128, n_experts=32,
                             k=8, act=ACT_SWIGLU, noisy=False, logit_bias="zipf1.1", seed=2104),
    # every expert kept (k == n): the load estimator's threshold is -inf for all
    "all_kept": MoEConfig("bwd_all_kept", T=130, d_model=64, d_hidden=64, n_experts=4, k=4,
                          expert_bias_std=0.1, seed=2105),
    # ReLU experts with a shared ReLU expert, noisy gate
    "relu_shared": MoEConfig("bwd_relu_shared", T=384, d_model=64, d_hidden=128, n_experts=8,
                             k=2, d_hidden_shared=128, seed=2106),
    # fp32 experts: the small correctness workload as it is, and one with
    # capacity drops and expert biases
    "tiny_f32": PRESETS["tiny_f32"],
    "f32_capacity": MoEConfig("bwd_f32_capacity", T=300, d_model=64, d_hidden=192, n_experts=8,
                              k=2, expert_dtype=DTYPE_F32, capacity_factor=0.9,
                              expert_bias_std=0.1, seed=2107),
    # the two-level layer: 8 groups of 8 (noisy), 4 groups of 16 (clean, fp32 experts)
    "two_level": MoEConfig("bwd_two_level", T=320, d_model=128, d_hidden=128, n_experts=64,
                           k=4, n_groups=8, k_groups=2, seed=2108),
    "two_level_clean_f32": MoEConfig("bwd_two_level_clean", T=200, d_model=64, d_hidden=64,
                                     n_experts=64, k=4, n_groups=4, k_groups=2, noisy=False,
                                     expert_dtype=DTYPE_F32, seed=2109),
    # a two-level layer with 128 experts per group (two per lane in the
    # secondary gates' backward)
    "two_level_wide": MoEConfig("bwd_two_level_wide", T=192, d_model=64, d_hidden=64,
                                n_experts=512, k=4, n_groups=4, k_groups=2, seed=300),
    # the gate backward's wide row layouts: 16 and 32 experts per lane
    "wide_gate": MoEConfig("bwd_wide_gate", T=256, d_model=64, d_hidden=64, n_experts=1024,
                           k=4, logit_bias="normal0.5", seed=2110),
    "widest_gate": MoEConfig("bwd_widest_gate", T=256, d_model=64, d_hidden=64,
                             n_experts=2048, k=8, logit_bias="normal0.5", seed=2110),
    # d_model >= 2048 with few gate tiles: the gate GEMM splits K in two
    # ([0, 1280) and [1280, 2112)), and the backward reads the logits the gate
    # epilogue summed from the partials
    "ksplit_noisy": MoEConfig("bwd_ksplit_noisy", T=256, d_model=2112, d_hidden=64,
                              n_experts=16, k=2, seed=2111),
    "ksplit_two_level": MoEConfig("bwd_ksplit_two_level", T=192, d_model=2048, d_hidden=64,
                                  n_experts=32, k=4, n_groups=4, k_groups=2, seed=2112),
}

GRAD_OF = dict(dw_gate="w_gate", db_gate="b_gate", dw_noise="w_noise", dw1="w1", db1="b1",
               dw3="w3", dw2="w2", db2="b2", dws1="ws1", dws3="ws3", dws2="ws2",
               dw_gate2="w_gate2", dw_noise2="w_noise2")


def _oracle_backward(cfg, h, dy, dl):
    if cfg.hierarchical:
        return oracle.backward_hier(
            h["x"], h["w_gate"], h.get("w_noise"), h.get("noise"), cfg.k_groups, h["w_gate2"],
            h.get("w_noise2"), h.get("noise2"), cfg.k2, h["w1"], h["w2"], dy, dl,
            b1=h.get("b1"), b2=h.get("b2"), bf16=cfg.expert_dtype != DTYPE_F32,
            w_importance=cfg.w_importance, w_load=cfg.w_load, alpha=cfg.alpha_switch,
            w_z=cfg.w_z, w_entropy=cfg.w_entropy)
    return oracle.backward(
        h["x"], h["w_gate"], cfg.k, h["w1"], h["w2"], dy, dl, b_gate=h.get("b_gate"),
        w_noise=h.get("w_noise"), noise=h.get("noise"), b1=h.get("b1"), w3=h.get("w3"),
        b2=h.get("b2"), mode=cfg.gate, act=cfg.act, bf16=cfg.expert_dtype != DTYPE_F32,
        capacity_factor=cfg.capacity_factor, w_importance=cfg.w_importance, w_load=cfg.w_load,
        alpha=cfg.alpha_switch, w_z=cfg.w_z, w_entropy=cfg.w_entropy, ws1=h.get("ws1"),
        ws3=h.get("ws3"), ws2=h.get("ws2"))


def _rank_k_unambiguous(H, k, rel=1e-4):
    """The k+1-th and k+2-th largest values of every row differ by more than
    rel * |value| (trivially true when fewer than k+2 experts exist)."""
    if H.shape[1] < k + 2:
        return True
    top = -np.sort(-H, axis=1)[:, k:k + 2]
    gap = top[:, 0] - top[:, 1]
    return bool(np.all(gap > rel * np.maximum(np.abs(top[:, 0]), np.abs(top[:, 1]))))


def _run(cfg, T=None):
    inp = make_inputs(cfg, device="cuda", T=T)
    dy, dl = make_grad_inputs(cfg, device="cuda", T=T)
    layer = MoELayer(cfg.replace(T=inp["x"].shape[0]), inp)
    torch.cuda.synchronize()
    g = layer.backward(inp["x"], dy, dl, inp.get("noise"), inp.get("noise2"))
    torch.cuda.synchronize()
    return inp, dy, dl, layer, {k: v.cpu().double().numpy() for k, v in g.items()}


def _compare(cfg, inp, dy, dl, got, check_rank_k=True):
    h = {k: to_numpy64(v) for k, v in inp.items() if v is not None}
    ref = _oracle_backward(cfg, h, to_numpy64(dy), to_numpy64(dl))
    if check_rank_k and h.get("w_noise") is not None and not cfg.hierarchical:
        assert _rank_k_unambiguous(ref["fwd"]["gate"].H, cfg.k), \
            "the case's inputs have a near-tie at rank k: pick another seed"
    tol = TOL_F32 if cfg.expert_dtype == DTYPE_F32 else TOL_BF16
    names = ["dx"] + [g for g, w in GRAD_OF.items() if w in h]
    if cfg.gate == GATE_SIGMOID_BIAS:
        names.remove("db_gate")
    for name in names:
        a = got[name]
        b = ref[name]
        assert a.shape == b.shape, name
        assert np.isfinite(a).all(), name
        sl = ref["slack"].get(name)
        if sl is None or not sl.any():
            err = max_abs_norm(a, b)
            log(f"  {name}: max-abs-normalised error {err:.2e}")
            assert err <= tol, (name, err)
            continue
        scale = np.max(np.abs(b))
        free = sl == 0
        err = float(np.max(np.abs(a - b)[free])) / scale if free.any() else 0.0
        log(f"  {name}: max-abs-normalised error {err:.2e} ({(~free).sum()} entries fed by "
            f"a ReLU mask at zero)")
        assert err <= tol, (name, err)
        over = np.abs(a - b) > sl + tol * scale
        assert not over.any(), (name, int(over.sum()))
    return ref


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_parity(case):
    cfg = CASES[case]
    log(f"[backward] {case}: T={cfg.T} d={cfg.d_model} h={cfg.d_hidden} n={cfg.n_experts} "
        f"k={cfg.k}")
    assert moe_gate_k_splits(cfg) == (2 if case.startswith("ksplit") else 1)
    inp, dy, dl, layer, got = _run(cfg)
    # the recomputed routing is the forward's: compare with the oracle's
    n, k, T = cfg.n_experts, cfg.k, cfg.T
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    layer.forward(inp["x"], inp.get("noise"), inp.get("noise2"), diag=dict(topk_idx=idx))
    torch.cuda.synchronize()
    ref = _compare(cfg, inp, dy, dl, got)
    orc_idx = ref["fwd"]["gate"]["topk_idx"] if cfg.hierarchical else ref["fwd"]["gate"].topk_idx
    np.testing.assert_array_equal(idx.cpu().numpy(), orc_idx)
    if cfg.capacity_factor > 0:
        assert (ref["fwd"]["dispatch"]["slot_pos"] < 0).any(), "the case should drop slots"


def test_backward_one_hot_many_tiles():
    """All gate weights zero: every logit ties, the lowest-index rule sends
    every token to experts 0 and 1, so those two experts' weight gradients
    run over all T rows (many K-steps) and every other expert's are zero."""
    cfg = MoEConfig("bwd_hot", T=700, d_model=64, d_hidden=128, n_experts=6, k=2, noisy=False,
                    expert_bias_std=0.1, seed=81)
    log("[backward] one-hot route T=700")
    inp = make_inputs(cfg, device="cuda")
    inp["w_gate"].zero_()
    dy, dl = make_grad_inputs(cfg, device="cuda")
    layer = MoELayer(cfg, inp)
    torch.cuda.synchronize()
    g = layer.backward(inp["x"], dy, dl)
    torch.cuda.synchronize()
    got = {k: v.cpu().double().numpy() for k, v in g.items()}
    for name in ("dw1", "dw2", "db1", "db2"):
        assert got[name][:2].any() and not got[name][2:].any(), name
    _compare(cfg, inp, dy, dl, got)


def test_backward_deterministic():
    cfg = CASES["lm_small"]
    _, _, _, _, a = _run(cfg)
    _, _, _, _, b = _run(cfg)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


def test_backward_empty_batch():
    """T = 0: no tokens, every weight gradient is zero."""
    cfg = CASES["relu_shared"]
    inp, dy, dl, layer, got = _run(cfg, T=0)
    assert got["dx"].shape == (0, cfg.d_model)
    for name, a in got.items():
        if name != "dx":
            assert not a.any(), name


def test_backward_upstream_losses_only():
    """dy = 0: only the auxiliary losses drive the gradients; the expert
    weights receive none."""
    cfg = CASES["lm_small"]
    inp = make_inputs(cfg, device="cuda")
    _, dl = make_grad_inputs(cfg, device="cuda")
    dy = torch.zeros((cfg.T, cfg.d_model), dtype=torch.float32, device="cuda")
    layer = MoELayer(cfg, inp)
    g = layer.backward(inp["x"], dy, dl, inp.get("noise"))
    torch.cuda.synchronize()
    got = {k: v.cpu().double().numpy() for k, v in g.items()}
    for name in ("dw1", "db1", "dw2", "db2"):
        assert not got[name].any(), name
    _compare(cfg, inp, dy, dl, got)


@pytest.mark.parametrize("name", ["lm_layer", "switch_cf", "hierarchical"])
def test_backward_full_size(name):
    """The whole workload at its full size, every gradient against the
    oracle's.  These batches hold a few tokens whose k+1-th and k+2-th gate
    values lie within 1e-4 of each other; the bar holds with them (their
    share of any gradient entry is small), so that check is not applied."""
    cfg = PRESETS[name]
    log(f"[backward] full size {name}: T={cfg.T} d={cfg.d_model} h={cfg.d_hidden} "
        f"n={cfg.n_experts} k={cfg.k}")
    inp, dy, dl, layer, got = _run(cfg)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    layer.forward(inp["x"], inp.get("noise"), inp.get("noise2"), diag=dict(topk_idx=idx))
    torch.cuda.synchronize()
    ref = _compare(cfg, inp, dy, dl, got, check_rank_k=False)
    orc_idx = ref["fwd"]["gate"]["topk_idx"] if cfg.hierarchical else ref["fwd"]["gate"].topk_idx
    np.testing.assert_array_equal(idx.cpu().numpy(), orc_idx)
