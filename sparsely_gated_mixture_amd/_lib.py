"""ctypes binding of libmoe.so (argument marshalling only).

Each function has the name and argument order of the C entry point in
include/moe.h.  Tensor arguments are torch tensors on the GPU (or None for an
optional pointer; plain integers are passed through as raw addresses).  The
stream defaults to torch's current HIP stream.  A non-OK status raises
MoEError carrying the library's message.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

EXPORTS = ["moe_workspace_size", "moe_expert_split_rows", "moe_gate_k_splits", "moe_expert_cu_split", "moe_fp8_weight_bytes", "moe_pack_fp8_weights", "moe_gate",
           "moe_gate_static", "moe_gate_hier", "moe_dispatch", "moe_expert_ffn", "moe_shared_ffn", "moe_combine",
           "moe_aux_loss", "moe_router_bias_update", "moe_forward",
           "moe_backward_workspace_size", "moe_backward", "moe_forward_train",
           "moe_backward_saved", "moe_status_string",
           "moe_last_error", "moe_probe_mfma", "moe_probe_hbm_read", "moe_profile_enable", "moe_profile_collect", "moe_profile_entry"]

N_LOSSES = 5  # importance, load, Switch, router z-loss, -gate entropy


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_hidden", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("k", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("act", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("k_groups", ctypes.c_int32),
                ("capacity_factor", ctypes.c_float), ("w_importance", ctypes.c_float),
                ("w_load", ctypes.c_float), ("alpha_switch", ctypes.c_float),
                ("w_z", ctypes.c_float), ("w_entropy", ctypes.c_float),
                ("d_hidden_shared", ctypes.c_int32)]


_vp = ctypes.c_void_p


class MoeWeights(ctypes.Structure):
    _fields_ = [("w_gate", _vp), ("b_gate", _vp), ("w_noise", _vp), ("w_gate2", _vp),
                ("w_noise2", _vp), ("w1", _vp), ("b1", _vp), ("w3", _vp), ("w2", _vp),
                ("b2", _vp), ("ws1", _vp), ("ws3", _vp), ("ws2", _vp)]


class MoeDiag(ctypes.Structure):
    _fields_ = [("topk_idx", _vp), ("topk_w", _vp), ("importance", _vp), ("load", _vp),
                ("counts_pre", _vp), ("counts", _vp), ("offsets", _vp), ("perm", _vp),
                ("slot_pos", _vp)]


class MoeGrads(ctypes.Structure):
    _fields_ = [("dx", _vp), ("dw_gate", _vp), ("db_gate", _vp), ("dw_noise", _vp),
                ("dw1", _vp), ("db1", _vp), ("dw3", _vp), ("dw2", _vp), ("db2", _vp),
                ("dws1", _vp), ("dws3", _vp), ("dws2", _vp), ("dw_gate2", _vp),
                ("dw_noise2", _vp)]


_lib = None


def load_library():
    """Load libmoe.so; fails loudly when the HIP library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    # MOE_LIBRARY_PATH: another build of the same sources (the sanitizer test
    # loads one whose host code carries AddressSanitizer / UBSan this way)
    path = os.environ.get("MOE_LIBRARY_PATH") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python sparsely_gated_mixture_amd/build.py`")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    S = ctypes.c_size_t
    cfgp = ctypes.POINTER(MoeConfig)
    L.moe_workspace_size.argtypes = [cfgp]
    L.moe_workspace_size.restype = S
    i32 = ctypes.c_int32
    L.moe_expert_split_rows.argtypes = [cfgp]
    L.moe_expert_split_rows.restype = ctypes.c_int32
    L.moe_gate_k_splits.argtypes = [cfgp]
    L.moe_gate_k_splits.restype = ctypes.c_int32
    L.moe_expert_cu_split.argtypes = [cfgp, P, i32, i32]
    L.moe_expert_cu_split.restype = ctypes.c_int32
    L.moe_fp8_weight_bytes.argtypes = [i32, i32, i32]
    L.moe_fp8_weight_bytes.restype = S
    L.moe_pack_fp8_weights.argtypes = [i32, i32, i32, i32, P, P, P]
    L.moe_pack_fp8_weights.restype = ctypes.c_int
    L.moe_gate.argtypes = [cfgp] + [P] * 10 + [P, S, P]
    L.moe_gate_static.argtypes = [cfgp] + [P] * 10 + [P]
    L.moe_gate_hier.argtypes = [cfgp] + [P] * 13 + [P, S, P]
    L.moe_dispatch.argtypes = [cfgp] + [P] * 8 + [P, S, P]
    L.moe_expert_ffn.argtypes = [cfgp] + [P] * 8 + [P, S, P]
    L.moe_shared_ffn.argtypes = [cfgp] + [P] * 5 + [P, S, P]
    L.moe_combine.argtypes = [cfgp] + [P] * 5 + [P]
    L.moe_aux_loss.argtypes = [cfgp] + [P] * 5 + [P]
    L.moe_router_bias_update.argtypes = [cfgp, P, P, ctypes.c_float, P]
    L.moe_forward.argtypes = [cfgp, ctypes.POINTER(MoeWeights)] + [P] * 5 + \
        [ctypes.POINTER(MoeDiag), P, S, P]
    L.moe_backward_workspace_size.argtypes = [cfgp]
    L.moe_backward_workspace_size.restype = S
    L.moe_backward.argtypes = [cfgp, ctypes.POINTER(MoeWeights)] + [P] * 5 + \
        [ctypes.POINTER(MoeGrads), P, S, P]
    L.moe_forward_train.argtypes = [cfgp, ctypes.POINTER(MoeWeights)] + [P] * 5 + [P, S, P]
    L.moe_backward_saved.argtypes = L.moe_backward.argtypes
    L.moe_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P,
                                 ctypes.POINTER(ctypes.c_double), P]
    L.moe_probe_mfma.restype = ctypes.c_int
    L.moe_probe_hbm_read.argtypes = [P, S, ctypes.c_int32, P, P]
    L.moe_probe_hbm_read.restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_profile_enable.argtypes = [ctypes.c_int]
    L.moe_profile_enable.restype = ctypes.c_int
    L.moe_profile_collect.argtypes = []
    L.moe_profile_collect.restype = ctypes.c_int
    L.moe_profile_entry.argtypes = [ctypes.c_int, ctypes.c_char_p, S,
                                    ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_longlong)]
    L.moe_profile_entry.restype = ctypes.c_int
    for name in ("moe_gate", "moe_gate_static", "moe_gate_hier", "moe_dispatch", "moe_expert_ffn", "moe_shared_ffn",
                 "moe_combine", "moe_aux_loss", "moe_router_bias_update", "moe_forward",
                 "moe_backward", "moe_forward_train", "moe_backward_saved"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def make_config(cfg) -> MoeConfig:
    """MoeConfig from anything with the moe_config field names (e.g. a
    workloads.MoEConfig)."""
    if isinstance(cfg, MoeConfig):
        return cfg
    return MoeConfig(int(cfg.T), int(cfg.d_model), int(cfg.d_hidden), int(cfg.n_experts),
                     int(cfg.k), int(cfg.gate), int(cfg.act), int(cfg.expert_dtype),
                     int(cfg.n_groups), int(cfg.k_groups), float(cfg.capacity_factor),
                     float(cfg.w_importance), float(cfg.w_load), float(cfg.alpha_switch),
                     float(getattr(cfg, "w_z", 1.0)), float(getattr(cfg, "w_entropy", 1.0)),
                     int(getattr(cfg, "d_hidden_shared", 0)))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _check(status: int):
    if status != MOE_OK:
        L = load_library()
        raise MoEError(status, (L.moe_last_error() or b"").decode())


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_last_error() -> str:
    return (load_library().moe_last_error() or b"").decode()


def moe_workspace_size(cfg) -> int:
    c = make_config(cfg)
    return load_library().moe_workspace_size(ctypes.byref(c))


def moe_fp8_weight_bytes(n_experts: int, N: int, K: int) -> int:
    return load_library().moe_fp8_weight_bytes(int(n_experts), int(N), int(K))


def moe_expert_split_rows(cfg) -> int:
    c = make_config(cfg)
    return int(load_library().moe_expert_split_rows(ctypes.byref(c)))


def moe_gate_k_splits(cfg) -> int:
    c = make_config(cfg)
    return int(load_library().moe_gate_k_splits(ctypes.byref(c)))


def moe_expert_cu_split(cfg, counts, cus: int = 0, product: int = 0) -> int:
    """counts: host int32 array (numpy or CPU tensor) of n_experts kept rows;
    product: 0 the first expert product, 1 the second."""
    import numpy as np
    c = make_config(cfg)
    a = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    return int(load_library().moe_expert_cu_split(ctypes.byref(c), a.ctypes.data, int(cus),
                                                  int(product)))


def moe_pack_fp8_weights(n_experts, N, K, src_dtype, src, dst, stream=None):
    _check(load_library().moe_pack_fp8_weights(int(n_experts), int(N), int(K), int(src_dtype),
                                               _ptr(src), _ptr(dst), _stream(stream)))


def moe_gate(cfg, x, w_gate, b_gate, w_noise, noise, topk_idx, topk_w, importance, load,
             gate_stats, ws, stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_gate(ctypes.byref(c), _ptr(x), _ptr(w_gate), _ptr(b_gate),
                                   _ptr(w_noise), _ptr(noise), _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(importance), _ptr(load), _ptr(gate_stats), wp, wb,
                                   _stream(stream)))


def moe_gate_static(cfg, x, w_gate, b_gate, w_noise, noise, topk_idx, topk_w, importance, load,
                    gate_stats, stream=None):
    c = make_config(cfg)
    _check(load_library().moe_gate_static(ctypes.byref(c), _ptr(x), _ptr(w_gate), _ptr(b_gate),
                                          _ptr(w_noise), _ptr(noise), _ptr(topk_idx),
                                          _ptr(topk_w), _ptr(importance), _ptr(load),
                                          _ptr(gate_stats), _stream(stream)))


def moe_gate_hier(cfg, x, w_gate, b_gate, w_noise, noise, w_gate2, w_noise2, noise2, topk_idx,
                  topk_w, importance, load, gate_stats, ws, stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_gate_hier(
        ctypes.byref(c), _ptr(x), _ptr(w_gate), _ptr(b_gate), _ptr(w_noise), _ptr(noise),
        _ptr(w_gate2), _ptr(w_noise2), _ptr(noise2), _ptr(topk_idx), _ptr(topk_w),
        _ptr(importance), _ptr(load), _ptr(gate_stats), wp, wb, _stream(stream)))


def moe_dispatch(cfg, topk_idx, x, counts_pre, counts, offsets, perm, slot_pos, x_perm, ws,
                 stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_dispatch(ctypes.byref(c), _ptr(topk_idx), _ptr(x),
                                       _ptr(counts_pre), _ptr(counts), _ptr(offsets),
                                       _ptr(perm), _ptr(slot_pos), _ptr(x_perm), wp, wb,
                                       _stream(stream)))


def moe_expert_ffn(cfg, x_perm, offsets, w1, b1, w3, w2, b2, y_perm, ws, stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_expert_ffn(ctypes.byref(c), _ptr(x_perm), _ptr(offsets), _ptr(w1),
                                         _ptr(b1), _ptr(w3), _ptr(w2), _ptr(b2), _ptr(y_perm),
                                         wp, wb, _stream(stream)))


def moe_shared_ffn(cfg, x, ws1, ws3, ws2, y_shared, ws, stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_shared_ffn(ctypes.byref(c), _ptr(x), _ptr(ws1), _ptr(ws3),
                                         _ptr(ws2), _ptr(y_shared), wp, wb, _stream(stream)))


def moe_combine(cfg, y_perm, slot_pos, topk_w, y_base, y, stream=None):
    c = make_config(cfg)
    _check(load_library().moe_combine(ctypes.byref(c), _ptr(y_perm), _ptr(slot_pos),
                                      _ptr(topk_w), _ptr(y_base), _ptr(y), _stream(stream)))


def moe_aux_loss(cfg, importance, load, counts_pre, gate_stats, losses, stream=None):
    c = make_config(cfg)
    _check(load_library().moe_aux_loss(ctypes.byref(c), _ptr(importance), _ptr(load),
                                       _ptr(counts_pre), _ptr(gate_stats), _ptr(losses),
                                       _stream(stream)))


def moe_router_bias_update(cfg, counts_pre, bias, gamma, stream=None):
    c = make_config(cfg)
    _check(load_library().moe_router_bias_update(ctypes.byref(c), _ptr(counts_pre), _ptr(bias),
                                                 float(gamma), _stream(stream)))


def make_weights(w_gate, b_gate=None, w_noise=None, w_gate2=None, w_noise2=None, w1=None,
                 b1=None, w3=None, w2=None, b2=None, ws1=None, ws3=None,
                 ws2=None) -> MoeWeights:
    return MoeWeights(_ptr(w_gate), _ptr(b_gate), _ptr(w_noise), _ptr(w_gate2), _ptr(w_noise2),
                      _ptr(w1), _ptr(b1), _ptr(w3), _ptr(w2), _ptr(b2), _ptr(ws1), _ptr(ws3),
                      _ptr(ws2))


def make_diag(**kw) -> MoeDiag:
    return MoeDiag(*[_ptr(kw.get(f)) for f, _ in MoeDiag._fields_])


def moe_forward(cfg, weights: MoeWeights, x, noise, noise2, y, losses, diag: MoeDiag | None, ws,
                stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_forward(ctypes.byref(c), ctypes.byref(weights), _ptr(x),
                                      _ptr(noise), _ptr(noise2), _ptr(y), _ptr(losses),
                                      ctypes.byref(diag) if diag is not None else None, wp, wb,
                                      _stream(stream)))


def moe_backward_workspace_size(cfg) -> int:
    c = make_config(cfg)
    return int(load_library().moe_backward_workspace_size(ctypes.byref(c)))


def make_grads(**kw) -> MoeGrads:
    return MoeGrads(*[_ptr(kw.get(f)) for f, _ in MoeGrads._fields_])


def moe_backward(cfg, weights: MoeWeights, x, noise, noise2, dy, dlosses, grads: MoeGrads, ws,
                 stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_backward(ctypes.byref(c), ctypes.byref(weights), _ptr(x),
                                       _ptr(noise), _ptr(noise2), _ptr(dy), _ptr(dlosses),
                                       ctypes.byref(grads), wp, wb, _stream(stream)))


def moe_forward_train(cfg, weights: MoeWeights, x, noise, noise2, y, losses, ws, stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_forward_train(ctypes.byref(c), ctypes.byref(weights), _ptr(x),
                                            _ptr(noise), _ptr(noise2), _ptr(y), _ptr(losses),
                                            wp, wb, _stream(stream)))


def moe_backward_saved(cfg, weights: MoeWeights, x, noise, noise2, dy, dlosses,
                       grads: MoeGrads, ws, stream=None):
    c = make_config(cfg)
    wp, wb = _ws(ws)
    _check(load_library().moe_backward_saved(ctypes.byref(c), ctypes.byref(weights), _ptr(x),
                                             _ptr(noise), _ptr(noise2), _ptr(dy),
                                             _ptr(dlosses), ctypes.byref(grads), wp, wb,
                                             _stream(stream)))


def moe_probe_mfma(dtype: int, blocks: int, iters: int, sink, stream=None) -> float:
    """Launch the matrix-unit peak probe; returns its flop count."""
    f = ctypes.c_double(0.0)
    _check(load_library().moe_probe_mfma(int(dtype), int(blocks), int(iters), _ptr(sink),
                                         ctypes.byref(f), _stream(stream)))
    return f.value


def moe_probe_hbm_read(buf, nbytes: int, blocks: int, sink, stream=None) -> None:
    """Launch the HBM read-stream probe over the first nbytes of buf."""
    _check(load_library().moe_probe_hbm_read(_ptr(buf), int(nbytes), int(blocks), _ptr(sink),
                                             _stream(stream)))


def moe_profile_enable(on: bool) -> None:
    _check(load_library().moe_profile_enable(1 if on else 0))


def moe_profile_collect() -> int:
    return load_library().moe_profile_collect()


def moe_profile_entry(i: int):
    """(kernel name, total milliseconds, launches) of collected entry i."""
    buf = ctypes.create_string_buffer(128)
    ms = ctypes.c_double()
    n = ctypes.c_longlong()
    _check(load_library().moe_profile_entry(i, buf, 128, ctypes.byref(ms), ctypes.byref(n)))
    return buf.value.decode(), ms.value, n.value
