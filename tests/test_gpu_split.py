"""Expert GEMMs split by size (bf16 experts with d_model and d_hidden both
>= 2048): experts that keep at least moe_expert_split_rows(cfg) rows run on
256 x 256 tiles, the rest on 128-row tiles.  Element-wise parity against the
oracle on shapes that reach both kernels, with an odd count of K-steps and
a K tail (chunks past K), N tails (a last N-tile of 8 or 40 columns), expert
biases through the big kernel's ReLU and identity epilogues, segments of one
to several 256-row tiles, the shared expert on 256-row tiles, and the
standalone moe_expert_ffn (which builds the two tile maps itself), and FP8
weights on both kernels (the oracle runs on the dequantized weights)."""
import numpy as np
import pytest
import torch

import oracle
import sparsely_gated_mixture_amd as moe
from sparsely_gated_mixture_amd.workloads import (ACT_SWIGLU, DTYPE_FP8, GATE_SIGMOID_BIAS,
                                                  MoEConfig, make_inputs)
from _support import (dev_inputs, expert_weights_host, full_parity, host, log, max_abs_norm)

pytestmark = pytest.mark.gpu


def _classes(cfg, counts):
    split = moe.moe_expert_split_rows(cfg)
    assert split > 0, "the case must reach the size split"
    small = int(np.sum((counts > 0) & (counts < split)))
    big = int(np.sum(counts >= split))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shares = [moe.moe_expert_cu_split(cfg, np.asarray(counts, np.int32), cus, prod)
              for prod in (0, 1)]
    log(f"  split at {split} rows: {small} experts on 128-row tiles, {big} on 256 x 256 "
        f"(largest {int(counts.max())} rows); side by side, 256 x 256 GEMM on {shares} of "
        f"{cus} CUs (first, second product)")
    if small and big and cfg.expert_dtype != DTYPE_FP8:
        assert all(0 < share < cus for share in shares)
    return split, small, big


def test_split_swiglu_sigmoid_shared():
    # d = 2112: 33 K-steps of 64 (an odd count: the big kernel runs one step
    # on zeros); h = 2056: the last 128-column N-tile of the SwiGLU GEMM holds
    # 8 columns.  Shared expert of width 2048 on 256-row tiles.
    cfg = MoEConfig("split_swiglu", T=400, d_model=2112, d_hidden=2056, n_experts=6, k=2,
                    act=ACT_SWIGLU, gate=GATE_SIGMOID_BIAS, noisy=False, logit_bias="zipf1.1",
                    d_hidden_shared=2048, seed=501)
    gpu, ref = full_parity(cfg)
    split, small, big = _classes(cfg, gpu["counts"])
    assert small >= 1 and big >= 1
    assert np.any(gpu["counts"] > 256)  # a segment of two 256-row tiles


def test_split_relu_biases_k_tail():
    # d = 2088: the last K-step holds 40 of 64 columns (chunks past K read as
    # zeros); the output GEMM's N = 2088 ends in a 40-column tile; expert
    # biases N(0, 0.1^2) through both kernels' epilogues.
    cfg = MoEConfig("split_relu", T=360, d_model=2088, d_hidden=2048, n_experts=5, k=2,
                    logit_bias="zipf1.1", expert_bias_std=0.1, seed=502)
    gpu, ref = full_parity(cfg)
    split, small, big = _classes(cfg, gpu["counts"])
    assert small >= 1 and big >= 1


def test_split_stage_expert_ffn():
    # moe_expert_ffn on its own: the tile maps are built inside the call.
    cfg = MoEConfig("split_stage", T=300, d_model=2048, d_hidden=2048, n_experts=4, k=2,
                    logit_bias="zipf1.1", seed=503)
    T, n, k, d = cfg.T, cfg.n_experts, cfg.k, cfg.d_model
    log(f"[stage expert_ffn, split] T={T} d={d} h={cfg.d_hidden} n={n}")
    inp = dev_inputs(cfg)
    h = host(inp, ["x", "w_gate", "b_gate", "w_noise", "noise"])
    g = oracle.gate(h["x"], h["w_gate"], k, h["b_gate"], h["w_noise"], h["noise"])
    disp = oracle.dispatch(g.topk_idx, n, 0.0)
    rows = disp["rows"]
    xp = torch.from_numpy(oracle.bf16_round(h["x"][disp["perm"]])).to(torch.bfloat16).to("cuda")
    xp = torch.cat([xp, torch.zeros((T * k - rows, d), dtype=torch.bfloat16, device="cuda")])
    off = torch.from_numpy(disp["offsets"]).to("cuda")
    yp = torch.full((T * k, d), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    moe.moe_expert_ffn(cfg, xp, off, inp["w1"], None, None, inp["w2"], None, yp, ws)
    torch.cuda.synchronize()
    _classes(cfg, disp["counts"])
    ew = expert_weights_host(inp, range(n))
    y_ref = oracle.experts_apply(h["x"], disp["perm"], disp["offsets"],
                                 np.stack([ew["w1"][e] for e in range(n)]),
                                 np.stack([ew["w2"][e] for e in range(n)]), bf16=True)
    err = max_abs_norm(yp[:rows].cpu().double().numpy(), y_ref)
    log(f"  y_perm error {err:.3e}")
    assert err <= 2e-2
    assert torch.all(yp[rows:] == 7.0)  # rows past offsets[n] untouched


def test_split_fp8_swiglu():
    # FP8 E4M3 weights on both kernels: h = 2112 ends the SwiGLU GEMM's last
    # 128-column N-tile with 64 columns (half the row pairs of the tile).
    cfg = MoEConfig("split_fp8_swiglu", T=400, d_model=2048, d_hidden=2112, n_experts=6, k=2,
                    act=ACT_SWIGLU, expert_dtype=DTYPE_FP8, noisy=False, logit_bias="zipf1.1",
                    seed=504)
    gpu, ref = full_parity(cfg)
    split, small, big = _classes(cfg, gpu["counts"])
    assert small >= 1 and big >= 1


def test_split_fp8_relu_biases():
    # FP8 weights with ReLU, expert biases N(0, 0.1^2) and the row scales in
    # the same epilogue; the output GEMM's N = 2112 ends in a 64-column tile.
    cfg = MoEConfig("split_fp8_relu", T=360, d_model=2112, d_hidden=2048, n_experts=5, k=2,
                    expert_dtype=DTYPE_FP8, logit_bias="zipf1.1", expert_bias_std=0.1, seed=505)
    gpu, ref = full_parity(cfg)
    split, small, big = _classes(cfg, gpu["counts"])
    assert small >= 1 and big >= 1


@pytest.mark.parametrize("case,counts", [
    # one big expert beside 31 small ones: the 256 x 256 GEMM gets a small share
    ("one_big", [130] + [3] * 31),
    # only big experts: the 128-row GEMM has no tiles, the other every CU
    ("all_big", [200, 150, 130, 140] + [0] * 28),
    # only small experts: the 256 x 256 GEMM has no tiles
    ("all_small", [5] * 20 + [0] * 12),
    # in between, with empty experts among the small ones
    ("mixed", [260, 140] + [10, 0] * 15),
])
def test_split_side_by_side_shares(case, counts):
    # moe_expert_ffn on hand-made segments whose CU shares span the range
    # (a few CUs to every CU for the big-expert GEMM); each expert's rows are
    # checked against the oracle's expert FFN.
    cfg = MoEConfig("split_shares", T=1024, d_model=2048, d_hidden=2048, n_experts=32, k=1,
                    seed=506)
    counts = np.asarray(counts, np.int32)
    n, d = cfg.n_experts, cfg.d_model
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shares = [moe.moe_expert_cu_split(cfg, counts, cus, prod) for prod in (0, 1)]
    log(f"[split shares] {case}: {rows} rows, 256 x 256 GEMM on {shares} of {cus} CUs "
        f"(first, second product)")
    want = {"all_big": cus, "all_small": 0}
    for share in shares:
        if case in want:
            assert share == want[case]
        elif case == "one_big":
            assert 8 <= share <= 24  # a small share: the big-expert GEMM on a few CUs per XCD
        else:
            assert 0 < share < cus
    inp = dev_inputs(cfg)
    r = np.random.default_rng(506)
    x = oracle.bf16_round(r.standard_normal((rows, d)))
    xp = torch.zeros((cfg.T * cfg.k, d), dtype=torch.bfloat16, device="cuda")
    xp[:rows] = torch.from_numpy(x).to(torch.bfloat16).to("cuda")
    yp = torch.full((cfg.T * cfg.k, d), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    moe.moe_expert_ffn(cfg, xp, torch.from_numpy(offsets).to("cuda"), inp["w1"], None, None,
                       inp["w2"], None, yp, ws)
    torch.cuda.synchronize()
    live = [e for e in range(n) if counts[e] > 0]
    ew = expert_weights_host(inp, live)
    w1 = np.zeros((n, cfg.d_hidden, d))
    w2 = np.zeros((n, d, cfg.d_hidden))
    for e in live:
        w1[e], w2[e] = ew["w1"][e], ew["w2"][e]
    y_ref = oracle.experts_apply(x, np.arange(rows), offsets, w1, w2, bf16=True, experts=live)
    err = max_abs_norm(yp[:rows].cpu().double().numpy(), y_ref)
    log(f"  y_perm error {err:.3e}")
    assert err <= 2e-2
    assert torch.all(yp[rows:] == 7.0)


def test_split_graph_replay_matches_eager():
    # The forward with the two size classes side by side (a second stream
    # forked from the caller's and joined back) captured into a HIP graph:
    # every replay, with eager work and synchronisations in between, equals
    # the eager result bit for bit.
    cfg = MoEConfig("split_graph", T=400, d_model=2048, d_hidden=2048, n_experts=6, k=2,
                    act=ACT_SWIGLU, noisy=False, logit_bias="zipf1.1", seed=507)
    inp = dev_inputs(cfg)
    layer = moe.MoELayer(cfg, inp)
    log("[split] graph replay, T=400, d=h=2048, 6 experts")
    y_ref, l_ref = layer.forward(inp["x"], inp["noise"])
    torch.cuda.synchronize()
    y_ref, l_ref = y_ref.clone(), l_ref.clone()
    y = torch.empty_like(y_ref)
    losses = torch.empty_like(l_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(inp["x"], inp["noise"], y=y, losses=losses)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(inp["x"], inp["noise"], y=y, losses=losses)
    for rep in range(4):
        y.fill_(float("nan"))
        losses.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}"
        assert torch.equal(losses, l_ref), f"replay {rep}"
        y2, _ = layer.forward(inp["x"], inp["noise"])
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref)


def test_split_two_host_threads():
    # Two host threads, each with its own layer, workspace and stream, run
    # side-by-side forwards at once (the library's second stream is shared
    # per device): every result equals the single-threaded one bit for bit.
    import threading
    cfg = MoEConfig("split_threads", T=400, d_model=2048, d_hidden=2048, n_experts=6, k=2,
                    act=ACT_SWIGLU, noisy=False, logit_bias="zipf1.1", seed=508)
    inp = dev_inputs(cfg)
    layers = [moe.MoELayer(cfg, inp) for _ in range(2)]
    log("[split] two host threads, T=400, d=h=2048, 6 experts")
    y_ref, l_ref = layers[0].forward(inp["x"], inp["noise"])
    torch.cuda.synchronize()
    y_ref, l_ref = y_ref.clone(), l_ref.clone()
    results, errors = [[], []], []

    def run(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(6):
                    y, l = layers[i].forward(inp["x"], inp["noise"])
                    results[i].append((y.clone(), l.clone()))
            st.synchronize()
        except Exception as exc:  # reported below
            errors.append(exc)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == 6
        for y, l in results[i]:
            assert torch.equal(y, y_ref) and torch.equal(l, l_ref)
