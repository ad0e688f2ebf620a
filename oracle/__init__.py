"""CPU oracle of the Sparsely-Gated MoE layer, forward and backward
(double precision).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only users.  The product path never
imports this package; it shares no code with the HIP implementation.

The arithmetic lives in ``oracle.c`` (built into ``liboracle.so`` next to this
file).  This module marshals numpy arrays and composes the stages in the order
the pages give them:

* gate: clean/noisy logits -> KeepTopK -> softmax (or the Switch router),
* the Importance and Load vectors and the auxiliary losses,
* dispatch into one merged batch per expert (with optional capacity),
* expert FFNs, gate-weighted combine,
* the two-level (hierarchical) composition,
* the backward pass of the flat layer (``backward``).

Citations use the page titles listed at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

GATE_TOPK_SOFTMAX = 0
GATE_SWITCH_TOP1 = 1
GATE_SIGMOID_BIAS = 2
ACT_RELU = 0
ACT_SWIGLU = 1
NEAR_TIE_REL = 1e-4

_dp = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_ip = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _opt(ptr_type):
    """ctypes argtype accepting None for optional arrays."""

    class _Opt:
        @classmethod
        def from_param(cls, obj):
            if obj is None:
                return None
            return ptr_type.from_param(obj)

    return _Opt


def num_threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Run the oracle's OpenMP loops on n threads (results do not depend on n)."""
    lib().oracle_set_num_threads(int(n))


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIBRARY_PATH: another build of oracle.c (the sanitizer test
        # loads an AddressSanitizer / UBSan build this way)
        path = os.environ.get("ORACLE_LIBRARY_PATH")
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build(force=True)
        L = ctypes.CDLL(path)
        c_int, c_dbl, c_i64 = ctypes.c_int, ctypes.c_double, ctypes.c_int64
        odp, oip = _opt(_dp), _opt(_ip)
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = c_int
        L.oracle_set_num_threads.argtypes = [c_int]
        L.oracle_set_num_threads.restype = None
        L.oracle_softplus.argtypes = [c_dbl]
        L.oracle_softplus.restype = c_dbl
        L.oracle_phi.argtypes = [c_dbl]
        L.oracle_phi.restype = c_dbl
        L.oracle_bf16_round.argtypes = [c_dbl]
        L.oracle_bf16_round.restype = c_dbl
        L.oracle_bf16_round_array.argtypes = [c_i64, _dp, _dp]
        L.oracle_gate_logits.argtypes = [c_int, c_int, c_int, _dp, _dp, odp, odp, odp, _dp, odp, _dp]
        L.oracle_keep_topk.argtypes = [c_int, c_int, c_int, _dp, _ip, odp, odp]
        L.oracle_gate_weights.argtypes = [c_int, c_int, c_int, c_int, _dp, _ip, _dp, odp]
        L.oracle_importance.argtypes = [c_int, c_int, _dp, _dp]
        L.oracle_load.argtypes = [c_int, c_int, c_int, _dp, _dp, _ip, _dp, _dp, odp, odp]
        L.oracle_dispatch.argtypes = [c_int, c_int, c_int, c_dbl, _ip, _ip, _ip, _ip, _ip, _ip]
        L.oracle_dispatch.restype = c_int
        L.oracle_expert_ffn.argtypes = [c_int, c_int, c_int, c_int, c_int, _dp, _dp, odp, odp, _dp,
                                        odp, _dp]
        L.oracle_combine.argtypes = [c_int, c_int, c_int, _dp, _ip, _dp, _dp]
        L.oracle_cv2.argtypes = [c_int, _dp]
        L.oracle_cv2.restype = c_dbl
        L.oracle_aux.argtypes = [c_int, c_int, c_int, _dp, odp, _ip, c_dbl, c_dbl, c_dbl, c_dbl,
                                 c_dbl, c_dbl, c_dbl, _dp]
        L.oracle_sigmoid_gate_weights.argtypes = [c_int, c_int, c_int, _dp, _ip, _dp, odp]
        L.oracle_zloss_sum.argtypes = [c_int, c_int, _dp]
        L.oracle_zloss_sum.restype = c_dbl
        L.oracle_entropy_sum.argtypes = [c_int, c_int, _dp]
        L.oracle_entropy_sum.restype = c_dbl
        L.oracle_bias_update.argtypes = [c_int, c_int, c_int, _ip, c_dbl, _dp]
        L.oracle_e4m3_decode.argtypes = [c_int]
        L.oracle_e4m3_decode.restype = c_dbl
        L.oracle_e4m3_encode.argtypes = [c_dbl]
        L.oracle_e4m3_encode.restype = c_int
        L.oracle_quantize_fp8_rows.argtypes = [c_int, c_int, _dp,
                                               np.ctypeslib.ndpointer(np.uint8, flags="C"), _dp]
        L.oracle_hier_load.argtypes = [c_int, c_int, _dp, _dp, _ip, _dp]
        L.oracle_cv2_grad.argtypes = [c_int, _dp, c_dbl, _dp]
        L.oracle_gate_backward.argtypes = [c_int, c_int, c_int, c_int, _dp, _dp, _dp, odp, odp,
                                           odp, _ip, _dp, _dp, _dp, _dp, _dp, _dp, odp, c_dbl,
                                           c_dbl, _dp, odp]
        _lib = L
    return _lib


def _d(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def softplus(z: float) -> float:
    return lib().oracle_softplus(float(z))


def phi(z: float) -> float:
    return lib().oracle_phi(float(z))


def bf16_round(a) -> np.ndarray:
    a = _d(a)
    out = np.empty_like(a)
    lib().oracle_bf16_round_array(a.size, a.reshape(-1), out.reshape(-1))
    return out


def cv2(v) -> float:
    v = _d(v)
    return lib().oracle_cv2(v.size, v)


# --------------------------------------------------------------------------
# stages
# --------------------------------------------------------------------------

def gate_logits(x, w_gate, b_gate=None, w_noise=None, noise=None):
    """clean, sp (None if noiseless), H  -- all [T, n] float64."""
    x, w_gate, b_gate, w_noise, noise = map(_d, (x, w_gate, b_gate, w_noise, noise))
    T, d = x.shape
    n = w_gate.shape[0]
    clean = np.empty((T, n))
    H = np.empty((T, n))
    sp = np.empty((T, n)) if w_noise is not None else None
    lib().oracle_gate_logits(T, d, n, x, w_gate, b_gate, w_noise, noise, clean, sp, H)
    return clean, sp, H


def keep_topk(H, k):
    H = _d(H)
    T, n = H.shape
    idx = np.empty((T, k), np.int32)
    hk = np.empty(T)
    hk1 = np.empty(T)
    lib().oracle_keep_topk(T, n, k, H, idx, hk, hk1)
    return idx, hk, hk1


def gate_weights(H, topk_idx, mode=GATE_TOPK_SOFTMAX):
    H = _d(H)
    topk_idx = _i(topk_idx)
    T, n = H.shape
    k = topk_idx.shape[1]
    w = np.empty((T, k))
    probs = np.empty((T, n))
    lib().oracle_gate_weights(T, n, k, mode, H, topk_idx, w, probs)
    return w, probs


def sigmoid_gate_weights(h, topk_idx):
    """[SURVEY] 6.2: kept weights s_i / sum s_j with s = Sigmoid(h), h the
    bias-free logits; also the dense gate vector."""
    h = _d(h)
    topk_idx = _i(topk_idx)
    T, n = h.shape
    k = topk_idx.shape[1]
    w = np.empty((T, k))
    probs = np.empty((T, n))
    lib().oracle_sigmoid_gate_weights(T, n, k, h, topk_idx, w, probs)
    return w, probs


def zloss_sum(Z) -> float:
    Z = _d(Z)
    return float(lib().oracle_zloss_sum(Z.shape[0], Z.shape[1] if Z.ndim == 2 else 0, Z))


def entropy_sum(G) -> float:
    G = _d(G)
    return float(lib().oracle_entropy_sum(G.shape[0], G.shape[1] if G.ndim == 2 else 0, G))


def bias_update(bias, counts_pre, T, k, gamma):
    """[SURVEY] 6.3 controller; returns the updated bias (float64)."""
    b = _d(bias).copy()
    c = _i(counts_pre)
    lib().oracle_bias_update(b.size, int(T), int(k), c, float(gamma), b)
    return b


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    L = lib()
    return np.array([L.oracle_e4m3_decode(int(v)) for v in c.reshape(-1)]).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float64)
    L = lib()
    return np.array([L.oracle_e4m3_encode(float(a)) for a in v.reshape(-1)],
                    dtype=np.uint8).reshape(v.shape)


def quantize_fp8_rows(w):
    """[SURVEY] section 9 read as FP8 E4M3 weights with a per-row scale:
    returns (codes uint8 [rows, K], scales float64 [rows])."""
    w = _d(w)
    rows, K = w.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty(rows)
    lib().oracle_quantize_fp8_rows(rows, K, w, codes, scales)
    return codes, scales


_E4M3_TABLE = None


def dequantize_fp8_rows(codes, scales) -> np.ndarray:
    """The values the codes stand for: decode(code) * scale of the row."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = e4m3_decode(np.arange(256))
    return _E4M3_TABLE[np.asarray(codes)] * np.asarray(scales, dtype=np.float64)[:, None]


def importance(probs):
    probs = _d(probs)
    T, n = probs.shape
    out = np.empty(n)
    lib().oracle_importance(T, n, probs, out)
    return out


def load(clean, sp, topk_idx, hk, hk1):
    clean, sp, hk, hk1 = map(_d, (clean, sp, hk, hk1))
    topk_idx = _i(topk_idx)
    T, n = clean.shape
    k = topk_idx.shape[1]
    P = np.empty((T, n))
    out = np.empty(n)
    lib().oracle_load(T, n, k, clean, sp, topk_idx, hk, hk1, P, out)
    return out, P


def dispatch(topk_idx, n, capacity_factor=0.0):
    topk_idx = _i(topk_idx)
    T, k = topk_idx.shape
    counts_pre = np.empty(n, np.int32)
    counts = np.empty(n, np.int32)
    offsets = np.empty(n + 1, np.int32)
    perm = np.zeros(max(T * k, 1), np.int32)
    slot_pos = np.empty((T, k), np.int32)
    rows = lib().oracle_dispatch(T, k, n, float(capacity_factor), topk_idx, counts_pre, counts,
                                 offsets, perm, slot_pos)
    return dict(counts_pre=counts_pre, counts=counts, offsets=offsets, perm=perm[:rows].copy(),
                slot_pos=slot_pos, rows=rows)


def expert_ffn(u, w1, w2, b1=None, w3=None, b2=None, act=ACT_RELU, bf16=False):
    """One expert on its merged rows u [rows, d]; returns [rows, d]."""
    u, w1, w2, b1, w3, b2 = map(_d, (u, w1, w2, b1, w3, b2))
    rows, d = u.shape
    h = w1.shape[0]
    y = np.empty((rows, d))
    if rows:
        lib().oracle_expert_ffn(rows, d, h, act, int(bool(bf16)), u, w1, b1, w3, w2, b2, y)
    return y


def combine(y_perm, slot_pos, topk_w, d):
    slot_pos = _i(slot_pos)
    topk_w = _d(topk_w)
    T, k = slot_pos.shape
    yp = _d(y_perm) if y_perm is not None and len(y_perm) else np.zeros((1, d))
    y = np.empty((T, d))
    lib().oracle_combine(T, k, d, yp, slot_pos, topk_w, y)
    return y


def aux(T, k, importance_v, load_v, counts_pre, w_importance, w_load, alpha, zsum=0.0,
        entsum=0.0, w_z=1.0, w_entropy=1.0):
    """The five losses: importance, load, Switch, z-loss, -entropy."""
    importance_v = _d(importance_v)
    load_v = _d(load_v)
    counts_pre = _i(counts_pre)
    out = np.empty(5)
    lib().oracle_aux(T, k, importance_v.size, importance_v, load_v, counts_pre,
                     float(w_importance), float(w_load), float(alpha), float(zsum),
                     float(entsum), float(w_z), float(w_entropy), out)
    return out


def hier_load(load_primary, load_secondary, group_tokens):
    load_primary, load_secondary = _d(load_primary), _d(load_secondary)
    a, b = load_secondary.shape
    out = np.empty(a * b)
    lib().oracle_hier_load(a, b, load_primary, load_secondary, _i(group_tokens), out)
    return out


def near_ties(hk, hk1):
    """O5: tokens whose k-th and (k+1)-th largest H differ by less than
    1e-4 * max(|a|, |b|) (never true when k == n)."""
    hk = np.asarray(hk)
    hk1 = np.asarray(hk1)
    with np.errstate(invalid="ignore"):
        return (hk - hk1) < NEAR_TIE_REL * np.maximum(np.abs(hk), np.abs(hk1))


# --------------------------------------------------------------------------
# compositions
# --------------------------------------------------------------------------

@dataclass
class GateResult:
    clean: np.ndarray
    sp: np.ndarray | None
    H: np.ndarray
    topk_idx: np.ndarray
    topk_w: np.ndarray
    probs: np.ndarray
    hk: np.ndarray
    hk1: np.ndarray
    importance: np.ndarray
    load: np.ndarray | None
    P: np.ndarray | None
    near_tie: np.ndarray
    zsum: float = 0.0       # sum over tokens of the squared norm of the softmax's logits
    entsum: float = 0.0     # sum over tokens of the gate distribution's entropy


def gate(x, w_gate, k, b_gate=None, w_noise=None, noise=None, mode=GATE_TOPK_SOFTMAX,
         route=None):
    """[PAPER] Noisy Top-K gating plus its Importance / Load vectors, the
    z-loss and entropy statistics ([WIKI] part 2).
    GATE_SIGMOID_BIAS ([SURVEY] 6.2, 6.3): selection on h + b, weights from
    Sigmoid(h) normalised over the kept experts; no noise, no Load; the
    z-loss statistic is taken over h (the bias is not a network output).
    route: optional [T, k] selection used in place of KeepTopK's (tests
    compare against another implementation's choice at near-ties); the
    weights, Importance and Load then follow from these logits with that
    selection held fixed, H_(k) and H_(k+1) still being the k-th and
    (k+1)-th largest values."""
    def select(H):
        idx, hk, hk1 = keep_topk(H, k)
        if route is not None:
            idx = _i(route)
            assert idx.shape == (H.shape[0], k)
        return idx, hk, hk1

    if mode == GATE_SIGMOID_BIAS:
        if w_noise is not None:
            raise ValueError("the sigmoid gate takes no noise")
        h, _, _ = gate_logits(x, w_gate)
        H = h + (_d(b_gate) if b_gate is not None else 0.0)
        idx, hk, hk1 = select(H)
        w, probs = sigmoid_gate_weights(h, idx)
        imp = importance(probs)
        return GateResult(H, None, H, idx, w, probs, hk, hk1, imp, None, None,
                          near_ties(hk, hk1), zloss_sum(h), entropy_sum(probs))
    clean, sp, H = gate_logits(x, w_gate, b_gate, w_noise, noise)
    idx, hk, hk1 = select(H)
    w, probs = gate_weights(H, idx, mode)
    imp = importance(probs)
    ld, P = (None, None)
    if sp is not None:
        ld, P = load(clean, sp, idx, hk, hk1)
    return GateResult(clean, sp, H, idx, w, probs, hk, hk1, imp, ld, P, near_ties(hk, hk1),
                      zloss_sum(H), entropy_sum(probs))


def experts_apply(x, perm, offsets, w1, w2, b1=None, w3=None, b2=None, act=ACT_RELU, bf16=False,
                  experts=None):
    """Run every (or the listed) expert on its merged rows; returns y_perm."""
    x = np.asarray(x)
    n = len(offsets) - 1
    rows = int(offsets[n])
    d = x.shape[1]
    y_perm = np.zeros((rows, d))
    for e in (range(n) if experts is None else experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        u = x[perm[lo:hi]]
        y_perm[lo:hi] = expert_ffn(u, w1[e], w2[e], None if b1 is None else b1[e],
                                   None if w3 is None else w3[e], None if b2 is None else b2[e],
                                   act, bf16)
    return y_perm


def forward(x, w_gate, k, w1, w2, *, b_gate=None, w_noise=None, noise=None, b1=None, w3=None,
            b2=None, mode=GATE_TOPK_SOFTMAX, act=ACT_RELU, bf16=False, capacity_factor=0.0,
            w_importance=0.1, w_load=0.1, alpha=1.0, w_z=1.0, w_entropy=1.0, ws1=None,
            ws3=None, ws2=None):
    """The whole flat layer: gate -> dispatch -> experts -> combine -> losses.
    ws1/ws3/ws2: the always-active shared expert ([SURVEY] 5.2, 6.2),
    y = E_shared(x) + sum_i g_i E_i(x)."""
    T, d = np.asarray(x).shape
    n = np.asarray(w_gate).shape[0]
    g = gate(x, w_gate, k, b_gate, w_noise, noise, mode)
    disp = dispatch(g.topk_idx, n, capacity_factor)
    y_perm = experts_apply(x, disp["perm"], disp["offsets"], w1, w2, b1, w3, b2, act, bf16)
    y = combine(y_perm, disp["slot_pos"], g.topk_w, d)
    y_shared = None
    if ws1 is not None:
        y_shared = expert_ffn(np.asarray(x), ws1, ws2, None, ws3, None, act, bf16)
        y = y_shared + y
    losses = aux(T, k, g.importance, g.load, disp["counts_pre"], w_importance, w_load, alpha,
                 g.zsum, g.entsum, w_z, w_entropy)
    return dict(gate=g, dispatch=disp, y_perm=y_perm, y=y, y_shared=y_shared, losses=losses)


def gate_hier(x, w_gate, w_noise, noise, k1, w_gate2, w_noise2, noise2, k2, b_gate=None,
              b_gate2=None, route=None):
    """O10 gating.  [NOTES] "分层 MoE": a primary gate picks k1 of a groups; in
    each chosen group a secondary gate (that group's own parameters) picks k2
    of its b experts.  Slot s*k2 + s2 of a token is expert g_s*b + e with
    weight w1_s * w2_{s,s2}.  Aux vectors: Importance over the product
    weights; Load in the factorised form of ``hier_load``.
    Shapes: w_gate2/w_noise2 [a, b, d], noise2 [T, k1, b].
    route: optional [T, k1*k2] combined selection held fixed in place of
    both levels' KeepTopK (see ``gate``)."""
    x = _d(x)
    T, d = x.shape
    w_gate2 = _d(w_gate2)
    a, b, _ = w_gate2.shape
    route = None if route is None else _i(route)
    pg = gate(x, w_gate, k1, b_gate, w_noise, noise,
              route=None if route is None else route[:, ::k2] // b)
    idx = np.empty((T, k1 * k2), np.int32)
    wts = np.empty((T, k1 * k2))
    near = pg.near_tie.copy()
    zsum = pg.zsum
    load_sec = np.zeros((a, b))
    group_tokens = np.zeros(a, np.int32)
    secondary = []  # (group, tokens, primary slots, GateResult) of each reached group
    noise2 = _d(noise2) if noise2 is not None else None
    w_noise2 = _d(w_noise2) if w_noise2 is not None else None
    for g in range(a):
        sel = np.nonzero(pg.topk_idx == g)  # (tokens ascending, slot)
        toks, slots = sel
        group_tokens[g] = len(toks)
        if len(toks) == 0:
            continue
        z2 = noise2[toks, slots] if noise2 is not None else None
        r2 = None
        if route is not None:
            r2 = np.stack([route[t, s * k2:(s + 1) * k2] % b for t, s in zip(toks, slots)])
        sg = gate(x[toks], w_gate2[g], k2, None if b_gate2 is None else b_gate2[g],
                  None if w_noise2 is None else w_noise2[g], z2, route=r2)
        secondary.append((g, toks, slots, sg))
        zsum += sg.zsum
        for r, (t, s) in enumerate(zip(toks, slots)):
            idx[t, s * k2:(s + 1) * k2] = g * b + sg.topk_idx[r]
            wts[t, s * k2:(s + 1) * k2] = pg.topk_w[t, s] * sg.topk_w[r]
            near[t] |= sg.near_tie[r]
        if sg.load is not None:
            load_sec[g] = sg.load
    n = a * b
    dense = np.zeros((T, n))
    for s in range(k1 * k2):
        dense[np.arange(T), idx[:, s]] = wts[:, s]
    imp = importance(dense)
    ld = hier_load(pg.load, load_sec, group_tokens) if pg.load is not None else None
    return dict(primary=pg, topk_idx=idx, topk_w=wts, importance=imp, load=ld,
                load_secondary=load_sec, group_tokens=group_tokens, near_tie=near,
                zsum=zsum, entsum=entropy_sum(dense), secondary=secondary)


def forward_hier(x, w_gate, w_noise, noise, k1, w_gate2, w_noise2, noise2, k2, w1, w2, *,
                 b1=None, b2=None, bf16=False, w_importance=0.1, w_load=0.1, alpha=1.0,
                 w_z=1.0, w_entropy=1.0):
    T, d = np.asarray(x).shape
    gh = gate_hier(x, w_gate, w_noise, noise, k1, w_gate2, w_noise2, noise2, k2)
    n = np.asarray(w_gate2).shape[0] * np.asarray(w_gate2).shape[1]
    disp = dispatch(gh["topk_idx"], n, 0.0)
    y_perm = experts_apply(x, disp["perm"], disp["offsets"], w1, w2, b1, None, b2, ACT_RELU, bf16)
    y = combine(y_perm, disp["slot_pos"], gh["topk_w"], d)
    losses = aux(T, k1 * k2, gh["importance"], gh["load"], disp["counts_pre"], w_importance,
                 w_load, alpha, gh["zsum"], gh["entsum"], w_z, w_entropy)
    return dict(gate=gh, dispatch=disp, y_perm=y_perm, y=y, losses=losses)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def cv2_grad(v, scale=1.0) -> np.ndarray:
    """scale * d CV(v)^2 / d v (population variance; 0 when the mean is 0)."""
    v = _d(v)
    out = np.empty(v.size)
    lib().oracle_cv2_grad(v.size, v, float(scale), out)
    return out


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


RELU_NEAR_ZERO = 2e-5  # |pre| at or below this fraction of sum |u_c w_jc| + |b_j|: either mask


def expert_ffn_backward(u, w1, w2, gout, b1=None, w3=None, b2=None, act=ACT_RELU, bf16=False,
                        slack=False):
    """Backward of one expert on its merged rows u [rows, d] (the forward of
    ``expert_ffn``), given gout = dL/d(expert output) [rows, d].  Returns
    (du, dw1, db1, dw3, dw2, db2); the absent parts are None.
    RELU: pre = u W1^T + b1, hid = max(0, pre), out = hid W2^T + b2:
      dW2 = gout^T hid, db2 = sum of gout rows, dhid = gout W2,
      dpre = dhid where pre > 0 else 0, dW1 = dpre^T u, db1 = sum of dpre rows,
      du = dpre W1.
    SWIGLU: hid = silu(a) * b with a = u W1^T, b = u W3^T:
      da = dhid * b * silu'(a), silu'(a) = s (1 + a (1 - s)) with s = Sigmoid(a),
      db = dhid * silu(a), dW1 = da^T u, dW3 = db^T u, du = da W1 + db W3.
    With bf16 the forward's rounded u and hid are the values used (the
    rounding itself is taken as the identity).
    ReLU'(0) is not defined, and a pre-activation within rounding of zero can
    take either mask value in an implementation that computes it in lower
    precision.  With slack=True a seventh value is returned: for ReLU, the
    largest change either choice can make, (s_du, s_dw1, s_db1), for the
    pre-activations with |pre| <= RELU_NEAR_ZERO * (sum_c |u_c w_jc| + |b_j|);
    None for SwiGLU (no discrete decision)."""
    u, w1, w2, gout, b1, w3, b2 = map(_d, (u, w1, w2, gout, b1, w3, b2))
    uq = bf16_round(u) if bf16 else u
    if act == ACT_SWIGLU:
        a = uq @ w1.T
        b = uq @ w3.T
        s = _sigmoid(a)
        hid = a * s * b
    else:
        pre = uq @ w1.T + (b1 if b1 is not None else 0.0)
        hid = np.maximum(pre, 0.0)
    hq = bf16_round(hid) if bf16 else hid
    dw2 = gout.T @ hq
    db2 = gout.sum(axis=0) if b2 is not None else None
    dhid = gout @ w2
    if act == ACT_SWIGLU:
        da = dhid * b * s * (1.0 + a * (1.0 - s))
        dbv = dhid * a * s
        return da @ w1 + dbv @ w3, da.T @ uq, None, dbv.T @ uq, dw2, db2
    dpre = np.where(pre > 0.0, dhid, 0.0)
    db1 = dpre.sum(axis=0) if b1 is not None else None
    out = (dpre @ w1, dpre.T @ uq, db1, None, dw2, db2)
    if not slack:
        return out
    mag = np.abs(uq) @ np.abs(w1).T + (np.abs(b1) if b1 is not None else 0.0)
    amb = np.where(np.abs(pre) <= RELU_NEAR_ZERO * mag, np.abs(dhid), 0.0)
    return out + ((amb @ np.abs(w1), amb.T @ np.abs(uq), amb.sum(axis=0)),)


def _combine_backward(dy, y_perm, slot_pos, topk_w, rows, d):
    """dG[t,s] = <dy_t, y_perm[row]> and the expert output gradients
    gout[row] = topk_w[t,s] * dy_t for the kept slots (dropped slots: 0)."""
    T, k = slot_pos.shape
    dG = np.zeros((T, k))
    gout = np.zeros((rows, d))
    for t in range(T):
        for s in range(k):
            r = slot_pos[t, s]
            if r < 0:
                continue
            dG[t, s] = dy[t] @ y_perm[r]
            gout[r] = topk_w[t, s] * dy[t]
    return dG, gout


def _experts_backward(x, disp, gout, w1, w2, w3, b1, b2, act, bf16):
    """Every expert's backward on its merged rows; returns (dx, grads, slack)
    with dx the tokens' input gradients summed in slot order."""
    T, d = x.shape
    n = w1.shape[0]
    h = w1.shape[1]
    offsets, perm, slot_pos = disp["offsets"], disp["perm"], disp["slot_pos"]
    rows = int(offsets[n])
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    dw3 = np.zeros_like(w3) if w3 is not None else None
    db1 = np.zeros((n, h)) if b1 is not None else None
    db2 = np.zeros((n, d)) if b2 is not None else None
    du_perm = np.zeros((rows, d))
    relu = act != ACT_SWIGLU
    slack_du = np.zeros((rows, d))
    slack = dict(dx=np.zeros((T, d)), dw1=np.zeros_like(w1),
                 db1=np.zeros((n, h)) if b1 is not None else None, dws1=None)
    for e in range(n):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        res = expert_ffn_backward(x[perm[lo:hi]], w1[e], w2[e], gout[lo:hi],
                                  None if b1 is None else b1[e],
                                  None if w3 is None else w3[e],
                                  None if b2 is None else b2[e], act, bf16, slack=relu)
        if relu:
            slack_du[lo:hi], slack["dw1"][e] = res[6][0], res[6][1]
            if b1 is not None:
                slack["db1"][e] = res[6][2]
        du_perm[lo:hi], dw1[e] = res[0], res[1]
        if db1 is not None:
            db1[e] = res[2]
        if dw3 is not None:
            dw3[e] = res[3]
        dw2[e] = res[4]
        if db2 is not None:
            db2[e] = res[5]
    dx = np.zeros((T, d))
    k = slot_pos.shape[1]
    for t in range(T):
        for s in range(k):
            r = slot_pos[t, s]
            if r >= 0:
                dx[t] += du_perm[r]
                slack["dx"][t] += slack_du[r]
    grads = dict(dw1=dw1, db1=db1, dw3=dw3, dw2=dw2, db2=db2)
    return dx, grads, slack


def _loss_coefficients(dl, T, k, n, importance_v, load_v, counts_pre, w_importance, w_load,
                       alpha, w_z, w_entropy):
    """dImportance = dl0 w_imp dCV^2 + dl2 alpha n f / T, dLoad = dl1 w_load
    dCV^2 (None without Load), and the z and entropy coefficients dl3 w_z / T
    and dl4 w_entropy / T (losses[4] = w_entropy / T * sum g ln g)."""
    f = np.asarray(counts_pre) / float(T * k)
    dimp = cv2_grad(importance_v, dl[0] * w_importance) + dl[2] * alpha * n * f / T
    dload = cv2_grad(load_v, dl[1] * w_load) if load_v is not None else None
    return dimp, dload, dl[3] * w_z / T, dl[4] * w_entropy / T


def _gate_backward(x, gr, k, mode, w_gate, w_noise, noise, dG, dimp, dload, c_z, c_ent):
    """oracle_gate_backward for one gate over the rows of x (GateResult gr);
    returns (dclean, draw or None)."""
    T, n = gr.H.shape
    noisy = gr.sp is not None
    if mode == GATE_SIGMOID_BIAS:
        Zs = x @ _d(w_gate).T        # the bias-free logits h
        clean = Zs
    else:
        Zs = gr.H
        clean = gr.clean
    raw = x @ _d(w_noise).T if noisy else None
    z = _d(noise) if noisy else None
    dclean = np.empty((T, n))
    draw = np.empty((T, n)) if noisy else None
    if T:
        lib().oracle_gate_backward(T, n, k, mode, _d(gr.H), _d(Zs), _d(clean),
                                   _d(gr.sp) if noisy else None, z, raw, _i(gr.topk_idx),
                                   _d(gr.topk_w), _d(gr.probs), _d(gr.hk), _d(gr.hk1),
                                   _d(dG), _d(dimp), _d(dload) if dload is not None else None,
                                   float(c_z), float(c_ent), dclean, draw)
    return dclean, draw


def backward(x, w_gate, k, w1, w2, dy, dlosses, *, b_gate=None, w_noise=None, noise=None,
             b1=None, w3=None, b2=None, mode=GATE_TOPK_SOFTMAX, act=ACT_RELU, bf16=False,
             capacity_factor=0.0, w_importance=0.1, w_load=0.1, alpha=1.0, w_z=1.0,
             w_entropy=1.0, ws1=None, ws3=None, ws2=None):
    """Gradients of L = sum_t <dy_t, y_t> + sum_j dlosses[j] * losses[j] for
    the flat layer of ``forward`` (same arguments), the routing held fixed.
    Returns a dict with dx, dw_gate, db_gate (None for the sigmoid gate,
    whose bias only moves the selection), dw_noise, dw1, db1, dw3, dw2, db2,
    dws1, dws3, dws2 (absent parts None), the forward's results ("fwd") and
    "slack": for ReLU experts, the largest change that either value of the
    mask at pre-activations within rounding of zero can make to dx, dw1, db1
    and dws1 (see expert_ffn_backward); zeros elsewhere.

    Stages, in reverse order of the forward ([PAPER] FAQ: the kept gate
    values are differentiable because the selection comes before the
    softmax; [NOTES] "Noisy Top-K Gating": the noise lets the load loss pass
    gradients):
      1. combine: dG[t,s] = <dy_t, y_perm[slot_pos[t,s]]> and the expert
         output rows receive topk_w[t,s] * dy_t (dropped slots neither);
      2. each expert (and the shared one, with weight 1) by
         ``expert_ffn_backward``; a token's input gradient sums its rows';
      3. the losses (``_loss_coefficients``);
      4. the gate by ``oracle_gate_backward`` (dclean, draw);
      5. the gate's linear maps: dW_g = dclean^T x, db = column sums of dclean,
         dW_noise = draw^T x, dx += dclean W_g + draw W_noise."""
    x = _d(x)
    T, d = x.shape
    w_gate = _d(w_gate)
    n = w_gate.shape[0]
    dy = _d(dy)
    dl = _d(dlosses)
    fwd = forward(x, w_gate, k, w1, w2, b_gate=b_gate, w_noise=w_noise, noise=noise, b1=b1,
                  w3=w3, b2=b2, mode=mode, act=act, bf16=bf16, capacity_factor=capacity_factor,
                  w_importance=w_importance, w_load=w_load, alpha=alpha, w_z=w_z,
                  w_entropy=w_entropy, ws1=ws1, ws3=ws3, ws2=ws2)
    g = fwd["gate"]
    disp = fwd["dispatch"]
    rows = int(disp["offsets"][n])

    # 1-2. combine and experts
    dG, gout = _combine_backward(dy, fwd["y_perm"], disp["slot_pos"], g.topk_w, rows, d)
    w1, w2, w3, b1, b2 = map(_d, (w1, w2, w3, b1, b2))
    dx, eg, slack = _experts_backward(x, disp, gout, w1, w2, w3, b1, b2, act, bf16)
    dws1 = dws3 = dws2 = None
    if ws1 is not None:
        relu = act != ACT_SWIGLU
        res = expert_ffn_backward(x, ws1, ws2, dy, None, ws3, None, act, bf16, slack=relu)
        dx += res[0]
        dws1, dws3, dws2 = res[1], res[3], res[4]
        if relu:
            slack["dx"] += res[6][0]
            slack["dws1"] = res[6][1]

    # 3-4. losses and gate
    dimp, dload, c_z, c_ent = _loss_coefficients(
        dl, T, k, n, g.importance, g.load, disp["counts_pre"], w_importance, w_load, alpha,
        w_z, w_entropy)
    dclean, draw = _gate_backward(x, g, k, mode, w_gate, w_noise, noise, dG, dimp, dload, c_z,
                                  c_ent)

    # 5. the gate's linear maps
    dw_gate = dclean.T @ x
    dx += dclean @ w_gate
    db_gate = None
    if b_gate is not None and mode != GATE_SIGMOID_BIAS:
        db_gate = dclean.sum(axis=0)
    dw_noise = None
    if draw is not None:
        dw_noise = draw.T @ x
        dx += draw @ _d(w_noise)
    return dict(dx=dx, dw_gate=dw_gate, db_gate=db_gate, dw_noise=dw_noise, dws1=dws1,
                dws3=dws3, dws2=dws2, dG=dG, dclean=dclean, draw=draw, fwd=fwd, slack=slack,
                **eg)


def backward_hier(x, w_gate, w_noise, noise, k1, w_gate2, w_noise2, noise2, k2, w1, w2, dy,
                  dlosses, *, b1=None, b2=None, bf16=False, w_importance=0.1, w_load=0.1,
                  alpha=1.0, w_z=1.0, w_entropy=1.0):
    """Gradients of L for the two-level layer of ``forward_hier`` (same
    arguments), the routing held fixed.  Returns dx, dw_gate, dw_noise,
    dw_gate2, dw_noise2 ([a, b, d]), dw1, db1, dw2, db2, "fwd" and "slack".

    The chain ([NOTES] "分层 MoE" for the structure; the readings of the
    two-level Importance and Load are those of the forward):
      1. combine and experts as for the flat layer, on the combined slots;
      2. the losses over Importance_H and Load_H, as for the flat layer;
      3. on each combined slot (s, s2) the gradient of the product weight
         w = w1_s * w2_{s,s2} is gw = dG + dImportance_H[expert] + c_ent (ln w
         + 1) (Importance_H and the entropy are taken over the products);
         then dw1_s = sum over s2 of gw * w2 and dw2_{s,s2} = gw * w1_s;
      4. Load_H[g*b+e] = Load_p[g] Load_g[e] / |X_g|: dLoad_p[g] = sum over e
         of dLoad_H * Load_g[e] / |X_g|, dLoad_g[e] = dLoad_H * Load_p[g] / |X_g|
         (0 when no token reaches g);
      5. the primary gate's backward with dG = dw1, no Importance or entropy
         term of its own, dLoad_p and the z coefficient; each group's secondary
         gate's backward over its rows likewise, with dw2 and dLoad_g;
      6. the linear maps of both levels (the secondary per group, over the
         rows routed to it)."""
    x = _d(x)
    T, d = x.shape
    dy = _d(dy)
    dl = _d(dlosses)
    w_gate2 = _d(w_gate2)
    a, b, _ = w_gate2.shape
    n = a * b
    k = k1 * k2
    fwd = forward_hier(x, w_gate, w_noise, noise, k1, w_gate2, w_noise2, noise2, k2, w1, w2,
                       b1=b1, b2=b2, bf16=bf16, w_importance=w_importance, w_load=w_load,
                       alpha=alpha, w_z=w_z, w_entropy=w_entropy)
    gh = fwd["gate"]
    disp = fwd["dispatch"]
    rows = int(disp["offsets"][n])

    # 1. combine and experts
    dG, gout = _combine_backward(dy, fwd["y_perm"], disp["slot_pos"], gh["topk_w"], rows, d)
    w1, w2, b1, b2 = map(_d, (w1, w2, b1, b2))
    dx, eg, slack = _experts_backward(x, disp, gout, w1, w2, None, b1, b2, ACT_RELU, bf16)

    # 2. losses
    dimp, dload, c_z, c_ent = _loss_coefficients(
        dl, T, k, n, gh["importance"], gh["load"], disp["counts_pre"], w_importance, w_load,
        alpha, w_z, w_entropy)

    # 3. product weights
    pg = gh["primary"]
    w2_of = np.zeros((T, k1, k2))  # secondary weights by (token, primary slot)
    for g, toks, slots, sg in gh["secondary"]:
        w2_of[toks, slots] = sg.topk_w
    dw1 = np.zeros((T, k1))
    dw2 = np.zeros((T, k1, k2))
    for t in range(T):
        for s in range(k1):
            for s2 in range(k2):
                j = s * k2 + s2
                wv = gh["topk_w"][t, j]
                gw = dG[t, j] + dimp[gh["topk_idx"][t, j]]
                if wv > 0.0:
                    gw += c_ent * (np.log(wv) + 1.0)
                dw1[t, s] += gw * w2_of[t, s, s2]
                dw2[t, s, s2] = gw * pg.topk_w[t, s]

    # 4. the factorised load
    dload_p = np.zeros(a) if dload is not None else None
    dload_g = np.zeros((a, b)) if dload is not None else None
    if dload is not None:
        cnt = gh["group_tokens"]
        lg = gh["load_secondary"]
        for g in range(a):
            if cnt[g] == 0:
                continue
            seg = dload[g * b:(g + 1) * b]
            dload_p[g] = (seg * lg[g]).sum() / cnt[g]
            dload_g[g] = seg * pg.load[g] / cnt[g]

    # 5-6. both gates
    zero_a, zero_b = np.zeros(a), np.zeros(b)
    dclean, draw = _gate_backward(x, pg, k1, GATE_TOPK_SOFTMAX, w_gate, w_noise, noise, dw1,
                                  zero_a, dload_p, c_z, 0.0)
    dw_gate = dclean.T @ x
    dx += dclean @ _d(w_gate)
    dw_noise = None
    if draw is not None:
        dw_noise = draw.T @ x
        dx += draw @ _d(w_noise)
    dw_gate2 = np.zeros_like(w_gate2)
    dw_noise2 = np.zeros_like(w_gate2) if w_noise2 is not None else None
    noise2 = _d(noise2) if noise2 is not None else None
    for g, toks, slots, sg in gh["secondary"]:
        xg = x[toks]
        z2 = noise2[toks, slots] if noise2 is not None else None
        dc2, dr2 = _gate_backward(xg, sg, k2, GATE_TOPK_SOFTMAX, w_gate2[g],
                                  None if w_noise2 is None else _d(w_noise2)[g], z2,
                                  dw2[toks, slots], zero_b,
                                  None if dload_g is None else dload_g[g], c_z, 0.0)
        dw_gate2[g] = dc2.T @ xg
        dx[toks] += dc2 @ w_gate2[g]
        if dr2 is not None:
            dw_noise2[g] = dr2.T @ xg
            dx[toks] += dr2 @ _d(w_noise2)[g]
    return dict(dx=dx, dw_gate=dw_gate, dw_noise=dw_noise, dw_gate2=dw_gate2,
                dw_noise2=dw_noise2, dG=dG, fwd=fwd, slack=slack, **eg)
