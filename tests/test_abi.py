"""The C ABI library loads, exports what include/moe.h declares, and rejects
bad arguments synchronously -- before any HIP call, so these run without a GPU."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import sparsely_gated_mixture_amd as moe
from sparsely_gated_mixture_amd import _lib
from sparsely_gated_mixture_amd.workloads import PRESETS, MoEConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = 0x10000  # an aligned non-null address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_calls():
    decl = declared_functions()
    for name in ["moe_gate", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_aux_loss",
                 "moe_forward", "moe_workspace_size", "moe_status_string", "moe_last_error",
                 "moe_gate_hier", "moe_shared_ffn", "moe_router_bias_update",
                 "moe_fp8_weight_bytes", "moe_pack_fp8_weights"]:
        assert name in decl
    assert sorted(_lib.EXPORTS) == decl


def test_library_exports_every_declared_symbol():
    L = moe.load_library()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name


def test_status_strings():
    for code in range(5):
        assert moe.moe_status_string(code)
    assert moe.moe_status_string(99) == "unknown status"


@pytest.mark.parametrize("name", list(PRESETS))
def test_workspace_size_of_presets(name):
    cfg = PRESETS[name]
    size = moe.moe_workspace_size(cfg)
    assert size > 0
    # the forward keeps x_perm and y_perm for every routed slot
    rows = cfg.T * cfg.k
    per = 4 if cfg.expert_dtype == 0 else 2  # x_perm is bf16 for bf16 and FP8 experts
    assert size >= rows * cfg.d_model * (per + 4)


def test_expert_cu_split():
    # The CU share of the 256 x 256-tile GEMM when the experts split by size
    # run side by side (a scheduling choice; results do not depend on it).
    fine = PRESETS["fine_swiglu"]
    n = fine.n_experts
    counts = np.zeros(n, np.int32)
    counts[:31] = 30808 // 31          # big experts (>= 128 rows)
    counts[31:161] = 2000 // 130       # small ones, 15 rows each
    share = moe.moe_expert_cu_split(fine, counts, 256)
    # First product: 31 x 1024 padded rows of 5.9e10 flops each (x W1^T and
    # x W3^T) at 5.13 TFLOP/s per CU, plus 31 M-tile groups of 58.7 MB of
    # W1 | W3 at 59 GB/s per CU, against 130 x 58.7 MB of small experts'
    # W1 | W3 at 30 GB/s per CU: 19.4 of 32 XCD rows, rounded to 19.  Second
    # product: 2.9e10 flops per row at 4.4 TFLOP/s against 130 x 29.4 MB of
    # W2: 20 of 32.
    assert share == 152
    assert moe.moe_expert_cu_split(fine, counts, 256, 1) == 160
    assert share % 8 == 0 and 8 <= share <= 248
    # product 0 or 1 only
    assert moe.moe_expert_cu_split(fine, counts, 256, 2) == -1
    assert moe.moe_expert_cu_split(fine, counts, 256, -1) == -1
    # the big experts count by whole 256-row tiles: 129 rows cost what 256 do
    c129, c256 = counts.copy(), counts.copy()
    c129[:31], c256[:31] = 129, 256
    for prod in (0, 1):
        assert (moe.moe_expert_cu_split(fine, c129, 256, prod) ==
                moe.moe_expert_cu_split(fine, c256, 256, prod))
    # no big expert: the small-expert GEMM keeps every CU; no small expert:
    # the big-expert GEMM does
    assert moe.moe_expert_cu_split(fine, np.full(n, 100, np.int32), 256) == 0
    assert moe.moe_expert_cu_split(fine, np.where(np.arange(n) < 8, 4096, 0).astype(np.int32),
                                   256) == 256
    # more rows on the big experts -> a larger share, never past 248
    prev = 0
    for rows in (200, 1000, 4000, 20000, 200000):
        c = counts.copy()
        c[:31] = rows
        cur = moe.moe_expert_cu_split(fine, c, 256)
        assert prev <= cur <= 248 and cur % 8 == 0
        prev = cur
    assert moe.moe_expert_cu_split(fine, np.where(np.arange(n) < 31, 10 ** 6, 1).astype(
        np.int32), 256) == 248
    # configs without the size split, FP8 weights (the two GEMMs run one
    # after the other), and bad arguments
    assert moe.moe_expert_cu_split(PRESETS["lm_layer"], np.full(256, 128, np.int32), 256) == 0
    assert moe.moe_expert_cu_split(PRESETS["fine_swiglu_fp8"], counts, 256) == 0
    assert moe.moe_expert_cu_split(fine, counts, -1) == -1


def test_gate_k_splits():
    # The gate GEMM's K-split: none while the tiles fill the CUs (three 64 x 64
    # or one 128 x 128 tile per CU; d_model >= 2048 takes 128 x 128) or
    # d_model < 2048; else up to ceil(768 / tiles) (256 / tiles for 128 x 128)
    # ranges of >= 1024, every range non-empty, the partial logits within 32 MiB.
    assert moe.moe_gate_k_splits(PRESETS["lm_layer"]) == 1          # d = 512
    assert moe.moe_gate_k_splits(PRESETS["fine_swiglu"]) == 4       # 64 tiles, 4 x 8 MiB
    assert moe.moe_gate_k_splits(PRESETS["sigmoid_shared"]) == 4
    assert moe.moe_gate_k_splits(base_cfg(T=700, d_model=3000, n_experts=96, k=4)) == 2
    assert moe.moe_gate_k_splits(base_cfg(T=64, d_model=8192, n_experts=8, k=2)) == 8
    # 768 tiles of 128 x 128 (T = 24576, 512 experts): no split
    assert moe.moe_gate_k_splits(base_cfg(T=24576, d_model=4096, n_experts=512, k=2)) == 1
    # T = 6144, d = 7168, 256 experts: 96 tiles, 2 x 12 MiB of partials
    assert moe.moe_gate_k_splits(base_cfg(T=6144, d_model=7168, n_experts=256, k=2)) == 2
    # a whole workspace per extra range: the size grows with the split
    one = moe.moe_workspace_size(base_cfg(T=64, d_model=1024, n_experts=8, k=2))
    eight = moe.moe_workspace_size(base_cfg(T=64, d_model=8192, n_experts=8, k=2))
    assert eight > one
    assert moe.moe_gate_k_splits(base_cfg(k=0)) == 0


def base_cfg(**kw):
    c = MoEConfig("t", T=64, d_model=32, d_hidden=64, n_experts=8, k=2)
    return c.replace(**kw)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=30), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_hidden=0), moe.MOE_ERR_INVALID_ARG),
    (dict(gate=7), moe.MOE_ERR_INVALID_ARG),
    (dict(gate=1, k=2), moe.MOE_ERR_INVALID_ARG),
    (dict(act=1, expert_dtype=0), moe.MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=5), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=4096, k=2), moe.MOE_ERR_UNSUPPORTED),  # flat gate limit
    (dict(n_groups=3), moe.MOE_ERR_INVALID_ARG),           # 8 % 3
    (dict(n_groups=2, k_groups=3), moe.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(gate=2, n_groups=2, k_groups=1), moe.MOE_ERR_INVALID_ARG),  # two-level: softmax gate
    (dict(d_hidden_shared=12), moe.MOE_ERR_INVALID_ARG),
    (dict(d_hidden_shared=-8), moe.MOE_ERR_INVALID_ARG),
    (dict(d_hidden_shared=16, expert_dtype=0), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_hidden_shared=16, n_groups=2, k_groups=1), moe.MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=2), moe.MOE_ERR_UNSUPPORTED),                  # d = 32: not a multiple of 64
    (dict(expert_dtype=2, d_model=64, d_hidden=128, d_hidden_shared=64), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_configs(kw, status):
    c = _lib.make_config(base_cfg(**kw))
    L = moe.load_library()
    assert L.moe_workspace_size(ctypes.byref(c)) == 0
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_combine(c, FAKE, FAKE, FAKE, None, FAKE, stream=0)
    assert ei.value.status == status
    assert moe.moe_last_error()


def test_null_and_misaligned_pointers():
    c = base_cfg()
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_combine(c, None, FAKE, FAKE, None, FAKE, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "y_perm" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_combine(c, FAKE + 4, FAKE, FAKE, None, FAKE, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "aligned" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:   # noisy gate without its noise tensor
        moe.moe_gate(c, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, None,
                     (FAKE, 1 << 30), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "noise" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:   # Switch router is noiseless
        moe.moe_gate(base_cfg(gate=1, k=1), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                     FAKE, None, (FAKE, 1 << 30), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoEError) as ei:   # flat call on a two-level config
        moe.moe_gate(base_cfg(n_groups=2, k_groups=1), FAKE, FAKE, None, None, None, FAKE, FAKE,
                     FAKE, None, None, (FAKE, 1 << 30), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_sigmoid_gate_shared_expert_and_bias_update_arguments():
    c = base_cfg(gate=2)
    with pytest.raises(moe.MoEError) as ei:   # the sigmoid gate is noiseless
        moe.moe_gate(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                     (FAKE, 1 << 30), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "sigmoid" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:   # no shared expert configured
        moe.moe_shared_ffn(c, FAKE, FAKE, None, FAKE, FAKE, (FAKE, 1 << 30), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    cs = base_cfg(d_hidden_shared=16, act=1)
    with pytest.raises(moe.MoEError) as ei:   # SwiGLU shared expert needs ws3
        moe.moe_shared_ffn(cs, FAKE, FAKE, None, FAKE, FAKE, (FAKE, 1 << 30), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "ws3" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:   # workspace sized without the shared expert
        moe.moe_shared_ffn(cs, FAKE, FAKE, FAKE, FAKE, FAKE,
                           (FAKE, moe.moe_workspace_size(base_cfg(act=1))), stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    w = moe.make_weights(FAKE, w1=FAKE, w2=FAKE, w3=FAKE)
    with pytest.raises(moe.MoEError) as ei:   # forward with a shared expert but no ws1
        moe.moe_forward(cs, w, FAKE, None, None, FAKE, FAKE, None,
                        (FAKE, moe.moe_workspace_size(cs)), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "ws1" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_router_bias_update(c, FAKE, None, 0.01, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "bias" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_router_bias_update(c, FAKE, FAKE, float("nan"), stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "gamma" in str(ei.value)
    assert moe.moe_workspace_size(cs) > moe.moe_workspace_size(base_cfg(act=1))


def test_fp8_sizes_and_arguments():
    assert moe.moe_fp8_weight_bytes(3, 64, 128) == 3 * (64 * 128 + 4 * 64)
    assert moe.moe_fp8_weight_bytes(1, 64, 100) == 0     # K % 64
    assert moe.moe_fp8_weight_bytes(1, 60, 128) == 0     # N % 8
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_pack_fp8_weights(1, 64, 100, 1, FAKE, FAKE, stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_pack_fp8_weights(1, 64, 128, 2, FAKE, FAKE, stream=0)   # src must be f32/bf16
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_pack_fp8_weights(1, 64, 128, 1, None, FAKE, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    ok = _lib.make_config(base_cfg(d_model=64, d_hidden=128, expert_dtype=2, act=1))
    assert moe.load_library().moe_workspace_size(ctypes.byref(ok)) > 0


def test_workspace_too_small_rejected_before_launch():
    c = base_cfg()
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_dispatch(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, (FAKE, 16), stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_expert_ffn(c, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, None, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    w = moe.make_weights(FAKE, w1=FAKE, w2=FAKE)
    size = moe.moe_workspace_size(c)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward(c, w, FAKE, None, None, FAKE, FAKE, None, (FAKE, size - 256), stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE


def test_gate_static_rejects_before_launch():
    # moe_gate_static (the library's own 48 MiB scratch): a config whose
    # gate needs more (logits [T, 2n] fp32: 65536 x 512 x 4 bytes) is
    # refused with MOE_ERR_WORKSPACE, an invalid config like moe_gate's --
    # both before any HIP call.
    big = base_cfg(T=65536, n_experts=256)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_gate_static(big, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                            stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    assert "scratch" in moe.moe_last_error()
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_gate_static(base_cfg(k=0), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            None, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_swiglu_requires_w3_and_no_bias():
    c = base_cfg(act=1)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_expert_ffn(c, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, (FAKE, 1 << 40),
                           stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "w3" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_expert_ffn(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, (FAKE, 1 << 40),
                           stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED


def test_mfma_probe_arguments():
    # Rejected before any launch: unsupported dtype, empty grid, missing sink.
    for args, what in [((moe.MOE_FP8, 1, 1, FAKE), "dtype"), ((moe.MOE_BF16, 0, 1, FAKE), "blocks"),
                       ((moe.MOE_F32, 1, 0, FAKE), "iters"), ((moe.MOE_BF16, 1, 1, None), "sink")]:
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_probe_mfma(*args, stream=0)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG and what in str(ei.value), args


def test_hbm_read_probe_arguments():
    for args, what in [((FAKE, 1024, 0, FAKE), "blocks"), ((FAKE, 8, 1, FAKE), "bytes"),
                       ((None, 1024, 1, FAKE), "buf"), ((FAKE, 1024, 1, None), "sink")]:
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_probe_hbm_read(*args, stream=0)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG and what in str(ei.value), args


def test_training_entry_points_validate_before_launch():
    # moe_backward, moe_forward_train and moe_backward_saved check every
    # pointer and the workspace before anything is enqueued.
    c = base_cfg(d_model=64, d_hidden=64)
    cc = _lib.make_config(c)
    L = moe.load_library()
    size = moe.moe_backward_workspace_size(c)
    assert size > moe.moe_workspace_size(c)
    # unsupported configurations report a zero backward workspace
    assert moe.moe_backward_workspace_size(base_cfg(d_model=64, d_hidden=128, expert_dtype=2)) == 0
    assert moe.moe_backward_workspace_size(base_cfg(d_model=96, d_hidden=64)) == 0
    w = moe.make_weights(FAKE, w_noise=FAKE, w1=FAKE, w2=FAKE)
    full = moe.make_grads(dx=FAKE, dw_gate=FAKE, dw_noise=FAKE, dw1=FAKE, dw2=FAKE)
    ws = (FAKE, size)
    # grads NULL
    st = L.moe_backward(ctypes.byref(cc), ctypes.byref(w), FAKE, FAKE, None, FAKE, FAKE, None,
                        FAKE, size, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "grads" in moe.moe_last_error()
    st = L.moe_backward_saved(ctypes.byref(cc), ctypes.byref(w), FAKE, FAKE, None, FAKE, FAKE,
                              None, FAKE, size, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "grads" in moe.moe_last_error()
    # a required gradient missing
    for call in (moe.moe_backward, moe.moe_backward_saved):
        with pytest.raises(moe.MoEError) as ei:
            call(c, w, FAKE, FAKE, None, FAKE, FAKE,
                 moe.make_grads(dx=FAKE, dw_gate=FAKE, dw_noise=FAKE, dw2=FAKE), ws, stream=0)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "dw1" in str(ei.value)
        with pytest.raises(moe.MoEError) as ei:   # noisy gate without its noise tensor
            call(c, w, FAKE, None, None, FAKE, FAKE, full, ws, stream=0)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "noise" in str(ei.value)
        with pytest.raises(moe.MoEError) as ei:   # workspace one byte short
            call(c, w, FAKE, FAKE, None, FAKE, FAKE, full, (FAKE, size - 1), stream=0)
        assert ei.value.status == moe.MOE_ERR_WORKSPACE
    # forward_train: y and losses are required; the backward workspace, not the forward's
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_train(c, w, FAKE, FAKE, None, None, FAKE, ws, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "y" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_train(c, w, FAKE, FAKE, None, FAKE, None, ws, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG and "losses" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_train(c, w, FAKE, FAKE, None, FAKE, FAKE,
                              (FAKE, moe.moe_workspace_size(c)), stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    # FP8 experts have no backward
    c8 = base_cfg(d_model=64, d_hidden=128, expert_dtype=2)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_train(c8, w, FAKE, FAKE, None, FAKE, FAKE, ws, stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
