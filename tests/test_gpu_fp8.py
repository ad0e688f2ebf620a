"""FP8 E4M3 expert weights on the GPU: the packing bit for bit against the
oracle's row quantization, and the layer forward (packed weights) against the
oracle run on the dequantized weights, at reduced and at full size."""
import numpy as np
import pytest
import torch

import oracle
import sparsely_gated_mixture_amd as moe
from sparsely_gated_mixture_amd.workloads import DTYPE_FP8, PRESETS, MoEConfig
from _support import (dev_inputs, full_parity, full_size_check, gpu_forward, log, max_abs_norm)

pytestmark = pytest.mark.gpu


def unpack(buf, n, N, K):
    """Codes [n, N, K] and scales [n, N] from the documented packed layout."""
    b = buf.cpu().numpy()
    per = N * K + 4 * N
    codes = np.empty((n, N, K), np.uint8)
    scales = np.empty((n, N), np.float32)
    for e in range(n):
        blk = b[e * per:e * per + N * K].reshape(N // 2, K // 64, 2, 64)
        codes[e] = blk.transpose(0, 2, 1, 3).reshape(N, K)
        scales[e] = b[e * per + N * K:(e + 1) * per].view(np.float32)
    return codes, scales


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pack_fp8_bit_exact(dtype):
    # Random rows, an all-zero row, and a row whose largest magnitude is 448
    # (scale exactly 1) holding every midpoint between E4M3 neighbours (the
    # rounding ties), negative midpoints and a negative zero.
    n, N, K = 3, 72, 192
    log(f"[fp8 pack] {dtype} n={n} N={N} K={K}")
    rng = np.random.default_rng(12)
    w = torch.from_numpy(rng.standard_normal((n, N, K)) * 0.05).to(dtype)
    w[0, 0] = 0
    mags = oracle.e4m3_decode(np.arange(0x7f))
    mids = (mags[:-1] + mags[1:]) / 2
    row = np.zeros(K)
    row[0] = 448.0
    row[1:1 + len(mids)] = mids
    row[1 + len(mids)] = -0.0
    rest = K - 2 - len(mids)
    row[2 + len(mids):] = -mids[:rest]
    w[1, 3] = torch.from_numpy(row).to(dtype)
    packed = moe.pack_fp8(w.cuda())
    torch.cuda.synchronize()
    assert packed.numel() == moe.moe_fp8_weight_bytes(n, N, K) == n * (N * K + 4 * N)
    codes, scales = unpack(packed, n, N, K)
    for e in range(n):
        oc, osc = oracle.quantize_fp8_rows(w[e].double().numpy())
        np.testing.assert_array_equal(codes[e], oc, err_msg=f"expert {e}")
        np.testing.assert_array_equal(scales[e], osc.astype(np.float32), err_msg=f"expert {e}")
    assert scales[1, 3] == 1.0 and scales[0, 0] == 1.0
    np.testing.assert_array_equal(codes[0, 0], 0)


def test_forward_fp8_lm_layer_ragged():
    full_parity(PRESETS["lm_layer_fp8"], T=1000)


def test_forward_fp8_swiglu_reduced_width():
    full_parity(PRESETS["fine_swiglu_fp8"].replace(d_model=256, d_hidden=128), T=512)


@pytest.mark.parametrize("bias", ["zero", "normal"])
def test_forward_fp8_odd_with_bias(bias):
    # n not a multiple of 8, a ragged last N tile (h = 192), expert biases
    # (all zero, or N(0, 0.1^2) so that a misplaced bias shows) through the
    # bias epilogue.
    kw = dict(zero_expert_bias=True) if bias == "zero" else dict(expert_bias_std=0.1)
    cfg = MoEConfig("fp8_odd", T=300, d_model=128, d_hidden=192, n_experts=37, k=3,
                    expert_dtype=DTYPE_FP8, seed=83, **kw)
    full_parity(cfg)


def test_full_size_fp8_lm_layer():
    full_size_check(PRESETS["lm_layer_fp8"], every_token=True)


def test_fp8_layer_close_to_bf16_layer():
    # The same inputs through bf16 and FP8 experts: the difference is the
    # weights' quantization (about 2^-4 relative per weight, averaging out
    # over the sums), far below the size of y.
    cfg = PRESETS["lm_layer"].replace(T=2048)
    inp = dev_inputs(cfg)
    log("[fp8 vs bf16] lm_layer T=2048")
    yb = gpu_forward(cfg, inp)["y"]
    yf = gpu_forward(cfg.replace(expert_dtype=DTYPE_FP8), inp)["y"]
    err = max_abs_norm(yf, yb)
    log(f"  FP8 vs bf16 experts: max-abs-normalised difference {err:.3e}")
    assert 1e-4 < err < 0.1
