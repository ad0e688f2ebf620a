"""Every workload preset at its full size on the GPU (through the C ABI),
checked against the oracle: routing of every token (bit-exact up to near
ties), dispatch bit-exact, importance / load / losses (the oracle held at the
GPU's routing where a near tie routes differently), and y element-wise --
on every token where the oracle's experts finish in seconds (lm_layer,
switch_cf, hierarchical), else on tokens that together cover every non-empty
expert, the hottest expert's last M-tile and every single-row expert."""
import numpy as np
import pytest
import torch

import oracle
import sparsely_gated_mixture_amd as moe
from sparsely_gated_mixture_amd.workloads import PRESETS, MoEConfig, make_inputs
from _support import (TOL_AUX, assert_close_rel, check_dispatch_exact, dev_inputs,
                      expert_weights_host, full_size_check, gpu_forward, host, log,
                      max_abs_norm, oracle_gate_any, oracle_gate_on_routing, y_tolerance)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,every_token", [("lm_layer", True), ("switch_cf", True),
                                              ("hierarchical", True), ("fine_swiglu", False),
                                              ("sigmoid_shared", False)])
def test_full_size(name, every_token):
    cfg = PRESETS[name]
    gpu = full_size_check(cfg, every_token=every_token)
    if name == "switch_cf":
        C = int(np.floor(cfg.capacity_factor * cfg.T * cfg.k / cfg.n_experts))
        assert np.all(gpu["counts"] <= C)
        dropped = np.mean(gpu["slot_pos"] < 0)
        log(f"  dropped fraction {dropped:.3f}")
        assert dropped > 0.1


def test_hierarchical_element_wise():
    # Two-level layer (a = b = 64 groups/experts, top-2 at each level) on 192
    # tokens, every output element against the oracle's two-level forward.
    cfg = PRESETS["hierarchical"]
    T = 192
    c = cfg.replace(T=T)
    log(f"[parity] hierarchical T={T}")
    inp = dev_inputs(c, T)
    gpu = gpu_forward(c, inp)
    h = host(inp)

    class Lazy:
        """Expert weights fetched from the device one expert at a time."""

        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return self.t[e].float().cpu().numpy()

    ref = oracle.forward_hier(h["x"], h["w_gate"], h["w_noise"], h["noise"], cfg.k_groups,
                              h["w_gate2"], h["w_noise2"], h["noise2"], cfg.k2, Lazy(inp["w1"]),
                              Lazy(inp["w2"]), bf16=True, w_importance=cfg.w_importance,
                              w_load=cfg.w_load, alpha=cfg.alpha_switch)
    gh = ref["gate"]
    bad = np.nonzero(np.any(gpu["topk_idx"] != gh["topk_idx"], axis=1))[0]
    assert all(gh["near_tie"][t] for t in bad) and len(bad) == 0
    np.testing.assert_allclose(gpu["topk_w"], gh["topk_w"], rtol=1e-4, atol=1e-6)
    check_dispatch_exact(c, gpu, T)
    assert max_abs_norm(gpu["y"], ref["y"]) <= y_tolerance(c)
    assert_close_rel(gpu["importance"], gh["importance"], 1e-5, 1e-5, "importance")
    assert_close_rel(gpu["load"], gh["load"], 1e-5, 1e-5, "load")
    assert_close_rel(gpu["losses"], ref["losses"], TOL_AUX, 1e-7, "losses")


@pytest.mark.parametrize("a,b", [(4, 128), (2, 256)])
def test_two_level_wide_groups_element_wise(a, b):
    # Secondary gates over 128 and 256 experts per group (two and four per
    # lane in the grouped top-k), every output element against the oracle.
    c = MoEConfig(f"hier_b{b}", T=192, d_model=64, d_hidden=64, n_experts=a * b, k=4,
                  n_groups=a, k_groups=2, seed=300)
    log(f"[parity] two-level a={a} b={b} T={c.T}")
    _two_level_check(c)


def test_two_level_gate_k_split_element_wise():
    # d_model = 2048 with 4 primary tiles: the primary gate's logit GEMM
    # splits K in two; every output element against the oracle.
    c = MoEConfig("hier_ksplit", T=256, d_model=2048, d_hidden=64, n_experts=32, k=4,
                  n_groups=4, k_groups=2, seed=812)
    assert moe.moe_gate_k_splits(c) == 2
    log(f"[parity] two-level, gate K-split: T={c.T} d={c.d_model}")
    _two_level_check(c)


def _two_level_check(c):
    inp = dev_inputs(c, c.T)
    gpu = gpu_forward(c, inp)
    h = host(inp)
    ew = expert_weights_host(inp, range(c.n_experts))
    ref = oracle.forward_hier(h["x"], h["w_gate"], h["w_noise"], h["noise"], c.k_groups,
                              h["w_gate2"], h["w_noise2"], h["noise2"], c.k2, ew["w1"], ew["w2"],
                              bf16=True, w_importance=c.w_importance, w_load=c.w_load,
                              alpha=c.alpha_switch)
    gh = ref["gate"]
    assert not np.any(gh["near_tie"]), "the case's inputs hold a near-tie: pick another seed"
    np.testing.assert_array_equal(gpu["topk_idx"], gh["topk_idx"])
    np.testing.assert_allclose(gpu["topk_w"], gh["topk_w"], rtol=1e-4, atol=1e-6)
    check_dispatch_exact(c, gpu, c.T)
    assert max_abs_norm(gpu["y"], ref["y"]) <= y_tolerance(c)
    assert_close_rel(gpu["importance"], gh["importance"], 1e-5, 1e-5, "importance")
    assert_close_rel(gpu["load"], gh["load"], 1e-5, 1e-5, "load")
    assert_close_rel(gpu["losses"], ref["losses"], TOL_AUX, 1e-7, "losses")


def test_stage_gate_hier():
    cfg = PRESETS["hierarchical"]
    T = 2048
    c = cfg.replace(T=T)
    log(f"[stage gate_hier] T={T}")
    small = c.replace(d_hidden=8)  # same gate seeds, tiny experts
    inp = make_inputs(small, device="cuda", T=T)
    n, k = c.n_experts, c.k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    imp = torch.empty(n, dtype=torch.float32, device="cuda")
    ld = torch.empty(n, dtype=torch.float32, device="cuda")
    st = torch.empty(2, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    moe.moe_gate_hier(c, inp["x"], inp["w_gate"], inp["b_gate"], inp["w_noise"], inp["noise"],
                      inp["w_gate2"], inp["w_noise2"], inp["noise2"], idx, w, imp, ld, st, ws)
    torch.cuda.synchronize()
    h = host(inp)
    oidx, ow, oimp, oload, _, near, zsum, entsum = oracle_gate_any(c, h)
    gi = idx.cpu().numpy()
    bad = np.nonzero(np.any(gi != oidx, axis=1))[0]
    assert all(near[t] for t in bad) and len(bad) <= 1e-4 * T
    ok = np.setdiff1d(np.arange(T), bad)
    np.testing.assert_allclose(w.cpu().numpy()[ok], ow[ok], rtol=1e-4, atol=1e-6)
    if len(bad):
        # the oracle held at the GPU's routing of the near-tie tokens
        oimp, oload, _, zsum, entsum = oracle_gate_on_routing(c, h, gi)
    assert_close_rel(imp.cpu().numpy(), oimp, 1e-5, 1e-5, "importance")
    assert_close_rel(ld.cpu().numpy(), oload, 1e-5, 1e-5, "load")
    assert_close_rel(st.cpu().numpy(), [zsum, entsum], TOL_AUX, 1e-7, "gate stats")
