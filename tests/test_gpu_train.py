"""The training step in two calls (moe_forward_train, then moe_backward_saved)
against the one-shot calls on the same seeded inputs.

moe_backward_saved reads the intermediates moe_forward_train kept, which are
those moe_backward recomputes with the same kernels in the same order, so its
gradients must equal moe_backward's bit for bit (moe_backward's own parity
with the oracle is tested elsewhere).  moe_forward_train's routing and losses
must equal moe_forward's bit for bit; y as well, except for SwiGLU bf16
experts, whose hidden value is formed from the two stored fp32
pre-activations by a separate kernel instead of the GEMM's epilogue: there y
must agree to 1e-3 max-abs-normalised (one bf16 rounding step of a few hidden
values at most, far inside the layer's bf16 bar).
"""
import numpy as np
import pytest
import torch

from _support import log, max_abs_norm
from sparsely_gated_mixture_amd import MoELayer
from sparsely_gated_mixture_amd.workloads import (ACT_SWIGLU, DTYPE_F32, PRESETS,
                                                  make_grad_inputs, make_inputs)
from test_gpu_backward import CASES

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().double().numpy()


def _check_step(cfg, T=None):
    inp = make_inputs(cfg, device="cuda", T=T)
    dy, dl = make_grad_inputs(cfg, device="cuda", T=T)
    cfg = cfg.replace(T=inp["x"].shape[0])
    x, noise, noise2 = inp["x"], inp.get("noise"), inp.get("noise2")
    layer = MoELayer(cfg, inp)
    y_ref, l_ref = layer.forward(x, noise, noise2)
    g_ref = layer.backward(x, dy, dl, noise, noise2)
    torch.cuda.synchronize()
    g_ref = {k: _np(v) for k, v in g_ref.items()}
    y_ref, l_ref = _np(y_ref), _np(l_ref)

    # the saved path, in a fresh layer (its own workspace)
    layer2 = MoELayer(cfg, inp)
    y, losses = layer2.forward_train(x, noise, noise2)
    g = layer2.backward(x, dy, dl, noise, noise2, saved=True)
    torch.cuda.synchronize()
    y, losses = _np(y), _np(losses)
    np.testing.assert_array_equal(losses, l_ref)
    if cfg.expert_dtype != DTYPE_F32:
        # moe_forward rounds bf16 experts' output rows to bf16 before the
        # combine (one rounding, 2^-9 relative, per kept slot); the training
        # forward keeps them in fp32 for the backward.
        err = max_abs_norm(y, y_ref) if y.size else 0.0
        log(f"  y vs moe_forward: {err:.2e} max-abs-normalised")
        assert err <= 4e-3, err
    else:
        np.testing.assert_array_equal(y, y_ref)
    assert g.keys() == g_ref.keys()
    for name, v in g.items():
        np.testing.assert_array_equal(_np(v), g_ref[name], err_msg=name)

    # a second backward over the same saved state (another upstream
    # gradient) equals the one-shot backward for that gradient
    dy2 = dy * -0.5
    g2 = layer2.backward(x, dy2, dl, noise, noise2, saved=True)
    g2_ref = layer.backward(x, dy2, dl, noise, noise2)
    torch.cuda.synchronize()
    for name, v in g2.items():
        np.testing.assert_array_equal(_np(v), _np(g2_ref[name]), err_msg=name)


@pytest.mark.parametrize("case", sorted(CASES))
def test_train_step_matches_one_shot(case):
    cfg = CASES[case]
    log(f"[train] {case}: T={cfg.T} d={cfg.d_model} h={cfg.d_hidden} n={cfg.n_experts} "
        f"k={cfg.k}")
    _check_step(cfg)


def test_train_step_empty_batch():
    log("[train] relu_shared at T=0")
    _check_step(CASES["relu_shared"], T=0)


@pytest.mark.parametrize("name", ["lm_layer", "hierarchical"])
def test_train_step_full_size(name):
    cfg = PRESETS[name]
    log(f"[train] full size {name}: T={cfg.T} d={cfg.d_model} h={cfg.d_hidden} "
        f"n={cfg.n_experts} k={cfg.k}")
    _check_step(cfg)
