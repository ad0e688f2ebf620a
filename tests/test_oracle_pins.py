"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, an invariant, a
brute-force enumeration, a library routine (scipy / numpy / torch CPU) or a
hand-worked example under tests/golden/ -- never against a retyped copy of its
own formula.  Citations name the page and section the fact comes from.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import ndtr

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Special values and library reductions (softplus, Phi, bf16)
# ---------------------------------------------------------------------------

def test_special_values():
    # Softplus(0) = ln 2; Phi(0) = 1/2
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=0, abs=1e-16)
    assert oracle.phi(0.0) == 0.5


def test_phi_matches_scipy_ndtr():
    # Phi against scipy's ndtr from z = -37 (just above ndtr's underflow) to 8.
    # Both sides evaluate erfc at a rounded -z/sqrt(2); the relative
    # sensitivity of erfc(y) to its argument is about 2*y^2, so the bound is a
    # few ulps times max(1, 2*y^2) per side.
    z = np.concatenate([np.linspace(-37, 8, 6001), [-20.0, -5.0, -1.0, 0.0, 1.0, 5.0]])
    ours = np.array([oracle.phi(v) for v in z])
    ref = ndtr(z)
    y = -z / np.sqrt(2.0)
    tol = 4 * np.maximum(1.0, 2 * y ** 2) * np.finfo(float).eps
    rel = np.abs(ours - ref) / ref
    assert np.all(rel <= tol), float(np.max(rel / tol))


def test_softplus_matches_logaddexp():
    z = np.concatenate([np.linspace(-60, 60, 2401), [-745.0, 700.0, 1e-12, -1e-12]])
    ours = np.array([oracle.softplus(v) for v in z])
    ref = np.logaddexp(0.0, z)
    np.testing.assert_allclose(ours, ref, rtol=1e-15, atol=1e-300)


def test_bf16_round_matches_torch():
    r = rng(0)
    vals = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (r.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, with both parities of bit 16
    bits = r.integers(0, 2**31, 4000, dtype=np.int64).astype(np.uint32)
    bits = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    bits = bits & np.uint32(0x7F7FFFFF)  # keep finite
    vals = np.concatenate([vals, bits.view(np.float32)])
    ours = oracle.bf16_round(vals.astype(np.float64))
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Hand-worked golden example
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "worked_layer.json")) as f:
        g = json.load(f)
    e = math.e
    ns = {"a": e / (1 + e), "b": 1 / (1 + e), "L": math.log(2.0),
          "Phi": lambda z: float(ndtr(z)), "log": math.log}

    def ev(v):
        if isinstance(v, list):
            return [ev(u) for u in v]
        if isinstance(v, str):
            return float(eval(v, {"__builtins__": {}}, ns))
        return v
    return g, ev


def test_golden_worked_layer():
    g, ev = _golden()
    inp, exp = g["inputs"], g["expected"]
    n, k, h = inp["n"], inp["k"], inp["h"]
    x = np.array(inp["x"], float)
    w_gate = np.array(inp["w_gate"])
    b_gate = np.array(inp["b_gate"])
    w_noise = np.array(inp["w_noise"], float)
    noise = np.array(ev(inp["noise"]))
    w1 = np.stack([(e + 1) * np.array(inp["w1_unit"], float) for e in range(n)])
    w2 = np.stack([np.array(inp["w2"], float)] * n)
    b1 = np.zeros((n, h))
    b2 = np.stack([[0.0, 0.0, float(e)] for e in range(n)])

    out = oracle.forward(x, w_gate, k, w1, w2, b_gate=b_gate, w_noise=w_noise, noise=noise,
                         b1=b1, b2=b2, alpha=1.0)
    gt = out["gate"]
    np.testing.assert_allclose(gt.H, ev(exp["H"]), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(gt.topk_idx, exp["topk_idx"])
    np.testing.assert_allclose(gt.topk_w, ev(exp["topk_w"]), rtol=1e-15)
    np.testing.assert_allclose(gt.importance, ev(exp["importance"]), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(gt.load, ev(exp["load"]), rtol=1e-14)
    d = out["dispatch"]
    np.testing.assert_array_equal(d["counts"], exp["counts"])
    np.testing.assert_array_equal(d["offsets"], exp["offsets"])
    np.testing.assert_array_equal(d["perm"], exp["perm"])
    np.testing.assert_array_equal(d["slot_pos"], exp["slot_pos"])
    np.testing.assert_allclose(out["y"], ev(exp["y"]), rtol=1e-15, atol=1e-15)
    assert out["losses"][2] == pytest.approx(ev(exp["switch_loss_alpha1"]), rel=1e-15)
    imp = np.array(ev(exp["importance"]))
    cv2 = np.mean((imp - imp.mean()) ** 2) / imp.mean() ** 2
    assert out["losses"][0] == pytest.approx(0.1 * cv2, rel=1e-14)
    assert out["losses"][3] == pytest.approx(ev(exp["zloss_mean"]), rel=1e-15)
    assert out["losses"][4] == pytest.approx(ev(exp["entropy_loss"]), rel=1e-14)

    cap = exp["capacity_1"]
    out = oracle.forward(x, w_gate, k, w1, w2, b_gate=b_gate, w_noise=w_noise, noise=noise,
                         b1=b1, b2=b2, capacity_factor=1.0)
    d = out["dispatch"]
    for key in ("counts_pre", "counts", "offsets", "perm", "slot_pos"):
        np.testing.assert_array_equal(d[key], cap[key], err_msg=key)
    np.testing.assert_allclose(out["y"], ev(cap["y"]), rtol=1e-15, atol=1e-15)


def test_golden_sigmoid_gate_shared_expert():
    """Selection-only bias, sigmoid weights normalised over the kept experts,
    the shared expert, the bias controller and the z / entropy losses, against
    the hand-worked tests/golden/sigmoid_gate.json."""
    with open(os.path.join(GOLDEN, "sigmoid_gate.json")) as f:
        g = json.load(f)

    def ev(v):
        if isinstance(v, list):
            return [ev(u) for u in v]
        if isinstance(v, str):
            return float(eval(v, {"__builtins__": {}}, {"log": math.log}))
        return v
    inp, exp = g["inputs"], g["expected"]
    n, k = inp["n"], inp["k"]
    x = np.array(inp["x"])
    w_gate = np.array(ev(inp["w_gate"]))
    bias = np.array(inp["bias"])
    w1 = np.stack([np.array(inp["w1_each"])] * n)
    w2 = np.stack([np.full((1, 2), float(e + 1)) for e in range(n)])
    out = oracle.forward(x, w_gate, k, w1, w2, b_gate=bias, mode=oracle.GATE_SIGMOID_BIAS,
                         ws1=np.array(inp["ws1"]), ws2=np.array(inp["ws2"]))
    gt = out["gate"]
    np.testing.assert_array_equal(gt.topk_idx, exp["topk_idx"])
    np.testing.assert_allclose(gt.topk_w, ev(exp["topk_w"]), rtol=1e-15)
    np.testing.assert_allclose(gt.importance, ev(exp["importance"]), rtol=1e-15, atol=1e-300)
    np.testing.assert_array_equal(out["dispatch"]["counts_pre"], exp["counts_pre"])
    np.testing.assert_allclose(out["y"], ev(exp["y"]), rtol=1e-15)
    assert out["losses"][3] == pytest.approx(ev(exp["zloss_mean"]), rel=1e-15)
    assert out["losses"][4] == pytest.approx(ev(exp["entropy_loss"]), rel=1e-14)
    nb = oracle.bias_update(bias, out["dispatch"]["counts_pre"], len(x), k, inp["gamma"])
    np.testing.assert_allclose(nb, ev(exp["bias_after"]), rtol=1e-15, atol=1e-18)


def test_sigmoid_gate_bias_selects_only():
    """[SURVEY] 6.3: the bias moves the selection, never the weights.  Adding
    a large bias to a fixed set of experts forces exactly that set; scaling
    the bias leaves the weights unchanged; the weights equal Sigmoid(h) of the
    kept experts over their sum (checked with scipy's expit)."""
    from scipy.special import expit
    rng = np.random.default_rng(11)
    T, d, n, k = 12, 6, 10, 3
    x = rng.standard_normal((T, d))
    w_gate = rng.standard_normal((n, d))
    forced = [7, 2, 5]
    bias = np.zeros(n)
    bias[forced] = [300.0, 200.0, 100.0]
    g1 = oracle.gate(x, w_gate, k, b_gate=bias, mode=oracle.GATE_SIGMOID_BIAS)
    g2 = oracle.gate(x, w_gate, k, b_gate=2 * bias, mode=oracle.GATE_SIGMOID_BIAS)
    np.testing.assert_array_equal(g1.topk_idx, np.tile(forced, (T, 1)))
    np.testing.assert_array_equal(g2.topk_idx, g1.topk_idx)
    np.testing.assert_allclose(g2.topk_w, g1.topk_w, rtol=0, atol=0)
    h = x @ w_gate.T
    s = expit(h[:, forced])
    np.testing.assert_allclose(g1.topk_w, s / s.sum(1, keepdims=True), rtol=1e-14)
    assert g1.load is None


def test_bias_update_controller_cases():
    """Counts above, at and below the even share T*k/n move the bias by -gamma,
    0, +gamma; a non-integral share (T*k/n = 2.5) puts 2 below and 3 above."""
    T, k, n = 10, 1, 4
    b = oracle.bias_update(np.zeros(n), [4, 2, 3, 1], T, k, 0.25)
    np.testing.assert_array_equal(b, [-0.25, 0.25, -0.25, 0.25])
    b = oracle.bias_update(np.ones(2), [5, 5], 5, 2, 0.5)
    np.testing.assert_array_equal(b, [1.0, 1.0])


def test_zloss_and_entropy_closed_forms():
    """Equal logits c: z statistic T*n*c^2, top-k weights 1/k (entropy ln k),
    Switch gate p = 1/n (entropy ln n), sigmoid gate 1/k; zero logits give a
    zero z statistic; doubling the logits multiplies it by 4."""
    T, d, n, k = 7, 3, 6, 2
    x = np.zeros((T, d))
    c = 0.75
    b = np.full(n, c)
    w = np.zeros((n, d))
    for mode, ent in ((oracle.GATE_TOPK_SOFTMAX, math.log(k)),
                      (oracle.GATE_SWITCH_TOP1, math.log(n))):
        kk = 1 if mode == oracle.GATE_SWITCH_TOP1 else k
        g = oracle.gate(x, w, kk, b_gate=b, mode=mode)
        assert g.zsum == pytest.approx(T * n * c * c, rel=1e-15)
        assert g.entsum == pytest.approx(T * ent, rel=1e-14)
    g = oracle.gate(x, w, k, b_gate=b, mode=oracle.GATE_SIGMOID_BIAS)
    assert g.zsum == 0.0            # the bias is not part of the network's logits
    assert g.entsum == pytest.approx(T * math.log(k), rel=1e-14)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((n, d))
    z1 = oracle.gate(x, w, k).zsum
    z2 = oracle.gate(x, 2 * w, k).zsum
    assert z2 == pytest.approx(4 * z1, rel=1e-14)


def test_hierarchical_equal_logits_entropy_adds():
    """Two-level gate with every logit equal: the product distribution is
    uniform over k1*k2 experts, so its entropy is ln k1 + ln k2 per token."""
    T, d, a, b, k1, k2 = 5, 2, 4, 3, 2, 2
    x = np.zeros((T, d))
    gh = oracle.gate_hier(x, np.zeros((a, d)), None, None, k1, np.zeros((a, b, d)), None, None,
                          k2)
    assert gh["entsum"] == pytest.approx(T * math.log(k1 * k2), rel=1e-14)
    assert gh["zsum"] == 0.0


def test_shared_expert_single_routed_expert():
    """n = k = 1 with the sigmoid gate (weight 1) plus a shared expert: y is
    the sum of two dense bf16 FFNs, computed here with numpy on the same
    bf16-rounded operands."""
    rng = np.random.default_rng(5)
    T, d, h = 9, 16, 24
    x = rng.standard_normal((T, d))
    r = lambda *s: oracle.bf16_round(rng.standard_normal(s) / 4)
    w1, w2 = r(1, h, d), r(1, d, h)
    ws1, ws2 = r(h, d), r(d, h)
    out = oracle.forward(x, rng.standard_normal((1, d)), 1, w1, w2, mode=oracle.GATE_SIGMOID_BIAS,
                         bf16=True, ws1=ws1, ws2=ws2)
    xb = oracle.bf16_round(x)
    ffn = lambda a, b: oracle.bf16_round(np.maximum(xb @ a.T, 0)) @ b.T
    np.testing.assert_allclose(out["gate"].topk_w, 1.0, rtol=0, atol=0)
    np.testing.assert_allclose(out["y"], ffn(w1[0], w2[0]) + ffn(ws1, ws2), rtol=1e-12,
                               atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force on tiny inputs (selection, kth_excluding, dispatch)
# ---------------------------------------------------------------------------

def _tiny_H(r, T, n, quant):
    H = r.standard_normal((T, n))
    if quant:
        H = np.round(H * 2) / 2  # many exact ties
        H[H == 0] = np.where(r.random(np.sum(H == 0)) < 0.5, -0.0, 0.0)
    return H


@pytest.mark.parametrize("quant", [False, True])
def test_keep_topk_brute_force(quant):
    r = rng(1 + quant)
    for n in range(1, 8):
        for k in range(1, n + 1):
            H = _tiny_H(r, 6, n, quant)
            idx, hk, hk1 = oracle.keep_topk(H, k)
            for t in range(H.shape[0]):
                v = H[t]
                valid = []
                for S in itertools.combinations(range(n), k):
                    rest = [j for j in range(n) if j not in S]
                    if not rest or min(v[list(S)]) >= max(v[rest]):
                        valid.append(S)
                best = min(valid)  # lowest indices win ties
                expect_order = sorted(best, key=lambda j: (-v[j], j))
                assert list(idx[t]) == expect_order
                # kth_excluding(H, k, i) by literally deleting i and sorting
                for i in range(n):
                    others = sorted(np.delete(v, i), reverse=True)
                    kth_ex = others[k - 1] if k - 1 < len(others) else -np.inf
                    thr = hk1[t] if i in best else hk[t]
                    assert thr == kth_ex


def test_load_against_deleted_kth():
    r = rng(3)
    T, d, n, k = 7, 5, 6, 2
    x = r.standard_normal((T, d))
    wg = r.standard_normal((n, d)) / math.sqrt(d)
    wn = r.standard_normal((n, d)) / math.sqrt(d)
    z = r.standard_normal((T, n))
    g = oracle.gate(x, wg, k, None, wn, z)
    raw = x @ wn.T
    sp = np.logaddexp(0.0, raw)
    clean = x @ wg.T
    H = clean + z * sp
    for t in range(T):
        for i in range(n):
            kth_ex = sorted(np.delete(H[t], i), reverse=True)[k - 1]
            assert g.P[t, i] == pytest.approx(ndtr((clean[t, i] - kth_ex) / sp[t, i]),
                                              rel=1e-12, abs=1e-15)
    np.testing.assert_allclose(g.load, g.P.sum(0), rtol=1e-14)


def _dispatch_brute(idx, n, cf):
    T, k = idx.shape
    cap = math.floor(cf * T * k / n) if cf > 0 else 10**9
    lists = [[] for _ in range(n)]
    dropped = set()
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            if len(lists[e]) < cap:
                lists[e].append((t, s))
            else:
                dropped.add((t, s))
    return lists, dropped, cap


@pytest.mark.parametrize("cf", [0.0, 0.5, 1.0, 1.25, 3.0, 1e30, 1e300])
def test_dispatch_brute_force(cf):
    r = rng(4)
    for (T, n, k) in [(1, 1, 1), (9, 4, 2), (33, 7, 3), (64, 5, 1), (40, 16, 4)]:
        idx = np.stack([r.permutation(n)[:k] for _ in range(T)]).astype(np.int32)
        if T > 3:
            idx[: T // 2, 0] = 0  # a hot expert to force drops
            for t in range(T // 2):
                row = list(idx[t])
                if row.count(0) > 1:
                    idx[t] = [0] + [e for e in r.permutation(np.arange(1, n))[: k - 1]]
        disp = oracle.dispatch(idx, n, cf)
        lists, dropped, cap = _dispatch_brute(idx, n, cf)
        counts = np.array([len(l) for l in lists])
        pre = np.bincount(idx.reshape(-1), minlength=n)
        np.testing.assert_array_equal(disp["counts_pre"], pre)
        np.testing.assert_array_equal(disp["counts"], counts)
        np.testing.assert_array_equal(disp["offsets"], np.concatenate([[0], np.cumsum(counts)]))
        perm = [t for l in lists for (t, s) in l]
        np.testing.assert_array_equal(disp["perm"], perm)
        row = 0
        expect_pos = -np.ones((T, k), np.int64)
        for l in lists:
            for (t, s) in l:
                expect_pos[t, s] = row
                row += 1
        np.testing.assert_array_equal(disp["slot_pos"], expect_pos)


def test_dispatch_invariants():
    # perm is a permutation of the kept pairs, slot_pos is its inverse, offsets
    # are monotone with offsets[n] = rows, tokens ascend inside each segment.
    r = rng(5)
    T, n, k = 500, 13, 3
    idx = np.stack([r.choice(n, k, replace=False, p=np.linspace(1, 3, n) / np.linspace(1, 3, n).sum())
                    for _ in range(T)]).astype(np.int32)
    for cf in (0.0, 0.8, 1.1):
        d = oracle.dispatch(idx, n, cf)
        off, perm, pos = d["offsets"], d["perm"], d["slot_pos"]
        assert np.all(np.diff(off) >= 0) and off[-1] == d["rows"] == d["counts"].sum()
        kept = [(t, s) for t in range(T) for s in range(k) if pos[t, s] >= 0]
        assert len(kept) == d["rows"]
        assert sorted(pos[pos >= 0].tolist()) == list(range(d["rows"]))
        for (t, s) in kept:
            p = pos[t, s]
            assert perm[p] == t
            e = idx[t, s]
            assert off[e] <= p < off[e + 1]
        for e in range(n):
            seg = perm[off[e]:off[e + 1]]
            assert np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def _ffn_np(u, w1, w2, b1=None, b2=None):
    hdn = u @ w1.T
    if b1 is not None:
        hdn = hdn + b1
    hdn = np.maximum(hdn, 0.0)
    y = hdn @ w2.T
    if b2 is not None:
        y = y + b2
    return y


def test_dense_softmax_mixture_when_k_equals_n():
    # k = n and no noise: G = softmax(clean) and y = sum_i softmax_i E_i(x)
    # ("soft routing", wiki article part 2), computed here with dense numpy.
    r = rng(6)
    T, d, n, h = 11, 6, 5, 7
    x = r.standard_normal((T, d))
    wg = r.standard_normal((n, d))
    bg = r.standard_normal(n)
    w1 = r.standard_normal((n, h, d))
    w2 = r.standard_normal((n, d, h))
    b1 = r.standard_normal((n, h))
    b2 = r.standard_normal((n, d))
    out = oracle.forward(x, wg, n, w1, w2, b_gate=bg, b1=b1, b2=b2)
    logits = x @ wg.T + bg
    sm = np.exp(logits - logits.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    dense = sum(sm[:, [i]] * _ffn_np(x, w1[i], w2[i], b1[i], b2[i]) for i in range(n))
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["gate"].probs, sm, rtol=1e-13)
    np.testing.assert_allclose(out["gate"].importance, sm.sum(0), rtol=1e-13)


def test_k_equals_n_load_and_counts():
    # k = n: kth_excluding is -inf for every expert, P = 1, Load_i = T,
    # CV^2(Load) = 0; every count is T and each segment is tokens 0..T-1.
    r = rng(7)
    T, d, n = 20, 4, 6
    x = r.standard_normal((T, d))
    g = oracle.gate(x, r.standard_normal((n, d)), n, None, r.standard_normal((n, d)),
                    r.standard_normal((T, n)))
    np.testing.assert_array_equal(g.load, np.full(n, float(T)))
    assert oracle.cv2(g.load) == 0.0
    d_ = oracle.dispatch(g.topk_idx, n)
    np.testing.assert_array_equal(d_["counts"], np.full(n, T))
    for e in range(n):
        np.testing.assert_array_equal(d_["perm"][d_["offsets"][e]:d_["offsets"][e + 1]],
                                      np.arange(T))


@pytest.mark.parametrize("k", [1, 2, 3])
def test_degenerate_all_equal_logits(k):
    # All-zero gate weights and noise: every H is equal, so by the
    # lowest-index rule every token takes experts 0..k-1 with weight 1/k.
    T, d, n = 10, 3, 5
    x = rng(8).standard_normal((T, d))
    zero = np.zeros((n, d))
    out = oracle.forward(x, zero, k, np.zeros((n, 2, d)), np.zeros((n, d, 2)), w_noise=zero,
                         noise=np.zeros((T, n)))
    g = out["gate"]
    np.testing.assert_array_equal(g.topk_idx, np.tile(np.arange(k), (T, 1)))
    np.testing.assert_allclose(g.topk_w, np.full((T, k), 1.0 / k), rtol=1e-15)
    np.testing.assert_array_equal(out["dispatch"]["counts"], [T] * k + [0] * (n - k))
    assert oracle.cv2(g.importance) == pytest.approx((n - k) / k, rel=1e-14)
    np.testing.assert_allclose(g.load, np.full(n, T / 2.0), rtol=1e-15)  # Phi(0) = 1/2
    assert out["losses"][1] == 0.0
    # capacity: exactly tokens 0..C-1 are kept by each of experts 0..k-1
    cf = 0.6
    C = math.floor(cf * T * k / n)
    dd = oracle.dispatch(g.topk_idx, n, cf)
    for e in range(k):
        np.testing.assert_array_equal(dd["perm"][dd["offsets"][e]:dd["offsets"][e + 1]],
                                      np.arange(C))
    assert np.all(dd["slot_pos"][C:] == -1)


def test_switch_degenerate_and_bounds():
    # Switch router with equal logits: p_i = 1/n, top-1 = expert 0, f_0 = 1,
    # P_i = 1/n -> n * sum f P = 1 (tufusi survey 3.2, minimum at uniform).
    T, d, n = 12, 3, 7
    x = rng(9).standard_normal((T, d))
    out = oracle.forward(x, np.zeros((n, d)), 1, np.zeros((n, 2, d)), np.zeros((n, d, 2)),
                         mode=oracle.GATE_SWITCH_TOP1, alpha=1.0)
    np.testing.assert_allclose(out["gate"].topk_w, 1.0 / n, rtol=1e-15)
    assert out["losses"][2] == pytest.approx(1.0, rel=1e-14)
    # random logits: the weight is the largest softmax probability, in [1/n, 1]
    r = rng(10)
    H = r.standard_normal((50, n)) * 3
    idx, _, _ = oracle.keep_topk(H, 1)
    w, p = oracle.gate_weights(H, idx, oracle.GATE_SWITCH_TOP1)
    sm = np.exp(H - H.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    np.testing.assert_allclose(w[:, 0], sm.max(1), rtol=1e-14)
    np.testing.assert_allclose(p, sm, rtol=1e-13)
    assert np.all(w >= 1.0 / n - 1e-15) and np.all(w <= 1.0)


def test_topk_weights_sum_to_one():
    r = rng(11)
    for k in (1, 2, 4, 8):
        H = r.standard_normal((40, 16)) * 4
        idx, _, _ = oracle.keep_topk(H, k)
        w, probs = oracle.gate_weights(H, idx)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
        assert np.all(w > 0) and np.all(w <= 1)
        assert np.all(np.diff(w, axis=1) <= 1e-15)  # slots in descending H
        # renormalised top-k of the full softmax (wiki article part 2)
        sm = np.exp(H - H.max(1, keepdims=True))
        sm /= sm.sum(1, keepdims=True)
        sel = np.take_along_axis(sm, idx, 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
        if k == 1:
            np.testing.assert_array_equal(w, 1.0)


def test_cv2_closed_forms():
    n, T = 9, 100.0
    assert oracle.cv2(np.full(n, T / n)) == pytest.approx(0.0, abs=1e-25)  # rounding of the mean only
    collapsed = np.zeros(n)
    collapsed[3] = T
    assert oracle.cv2(collapsed) == pytest.approx(n - 1, rel=1e-14)
    assert oracle.cv2(np.zeros(n)) == 0.0
    v = np.array([1.0, 2.0, 3.0, 6.0])
    assert oracle.cv2(v) == pytest.approx(np.var(v) / np.mean(v) ** 2, rel=1e-14)


def test_switch_loss_closed_forms():
    n, T = 8, 64
    uni = np.full(n, T // n, np.int32)
    l = oracle.aux(T, 1, np.full(n, T / n), None, uni, 0.1, 0.1, 1.0)
    assert l[2] == pytest.approx(1.0, rel=1e-14)
    col = np.zeros(n, np.int32)
    col[0] = T
    imp = np.zeros(n)
    imp[0] = T
    l = oracle.aux(T, 1, imp, None, col, 0.1, 0.1, 1.0)
    assert l[2] == pytest.approx(float(n), rel=1e-14)
    assert l[0] == pytest.approx(0.1 * (n - 1), rel=1e-14)


def test_single_expert_reduces_to_dense_ffn_bf16():
    # n = 1, k = 1: y = FFN(x), with bf16-rounded operands (torch's RNE
    # conversion) and a float64 numpy FFN.
    r = rng(12)
    T, d, h = 37, 24, 40
    x = r.standard_normal((T, d))
    wg = r.standard_normal((1, d))

    def bf(a):
        return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
    w1 = bf(r.standard_normal((1, h, d)) / math.sqrt(d))
    w2 = bf(r.standard_normal((1, d, h)) / math.sqrt(h))
    out = oracle.forward(x, wg, 1, w1, w2, bf16=True)
    xb = bf(x)
    hid = bf(np.maximum(xb @ w1[0].T, 0.0))
    np.testing.assert_allclose(out["y"], hid @ w2[0].T, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out["gate"].topk_w, 1.0)


def test_swiglu_expert_against_numpy():
    r = rng(13)
    rows, d, h = 9, 8, 12
    u = r.standard_normal((rows, d))
    w1 = r.standard_normal((h, d))
    w3 = r.standard_normal((h, d))
    w2 = r.standard_normal((d, h))
    y = oracle.expert_ffn(u, w1, w2, w3=w3, act=oracle.ACT_SWIGLU)
    g = u @ w1.T
    ref = ((g / (1.0 + np.exp(-g))) * (u @ w3.T)) @ w2.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Statistical semantics of P(x, i)  (Monte Carlo)
# ---------------------------------------------------------------------------

def test_load_probability_monte_carlo():
    # P(x,i) is the probability that expert i stays in the top k when only its
    # own noise z_i is redrawn: Pr[clean_i + z_i sp_i beats the k-th best of
    # the others].  The selection here is a full top-k per draw.
    r = rng(14)
    d, n, k = 6, 8, 2
    x = r.standard_normal((1, d))
    wg = r.standard_normal((n, d)) / math.sqrt(d)
    wn = r.standard_normal((n, d)) / math.sqrt(d)
    z = r.standard_normal((1, n))
    g = oracle.gate(x, wg, k, None, wn, z)
    clean, sp, H = g.clean[0], g.sp[0], g.H[0]
    draws = 1_000_000
    mc_r = np.random.default_rng(15)
    for i in range(n):
        zi = mc_r.standard_normal(draws)
        Hi = clean[i] + zi * sp[i]
        others = np.delete(H, i)
        beaten_by = (others[None, :] > Hi[:, None]).sum(1)
        frac = np.mean(beaten_by < k)
        assert abs(frac - g.P[0, i]) < 3e-3, (i, frac, g.P[0, i])


# ---------------------------------------------------------------------------
# Hierarchical composition
# ---------------------------------------------------------------------------

def test_hierarchical_one_group_reduces_to_flat():
    # a = 1, k1 = 1: the primary gate is 1 with Load_primary = T and
    # |X_0| = T, so the two-level layer is the flat layer over b experts.
    r = rng(16)
    T, d, b, k2, h = 25, 6, 7, 2, 5
    x = r.standard_normal((T, d))
    wg1 = r.standard_normal((1, d))
    wn1 = r.standard_normal((1, d))
    z1 = r.standard_normal((T, 1))
    wg2 = r.standard_normal((1, b, d))
    wn2 = r.standard_normal((1, b, d))
    z2 = r.standard_normal((T, 1, b))
    w1 = r.standard_normal((b, h, d))
    w2 = r.standard_normal((b, d, h))
    hier = oracle.forward_hier(x, wg1, wn1, z1, 1, wg2, wn2, z2, k2, w1, w2)
    flat = oracle.forward(x, wg2[0], k2, w1, w2, w_noise=wn2[0], noise=z2[:, 0])
    np.testing.assert_allclose(hier["y"], flat["y"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(hier["gate"]["importance"], flat["gate"].importance, rtol=1e-14)
    np.testing.assert_allclose(hier["gate"]["load"], flat["gate"].load, rtol=1e-14)
    np.testing.assert_array_equal(hier["gate"]["topk_idx"], flat["gate"].topk_idx)
    sel = [0, 1, 2, 4]
    np.testing.assert_allclose(hier["losses"][sel], flat["losses"][sel], rtol=1e-12, atol=1e-15)
    # The z-loss statistic covers both gating networks: with one group the
    # primary gate's single logit per token is the only extra term.
    T = len(hier["y"])
    prim = hier["gate"]["primary"].H
    np.testing.assert_allclose(hier["losses"][3], flat["losses"][3] + float(np.sum(prim * prim)) / T,
                               rtol=1e-12)


def test_gate_route_held_fixed():
    """gate(route=...) holds a given selection: with the oracle's own
    selection every output is unchanged; with a near-tie swapped the weights
    are the softmax over the chosen values, Importance still sums to T, and
    Load changes only for the swapped experts."""
    r = rng(21)
    T, d, n, k = 40, 8, 9, 3
    x = r.standard_normal((T, d))
    wg, wn = r.standard_normal((n, d)), r.standard_normal((n, d))
    z = r.standard_normal((T, n))
    g = oracle.gate(x, wg, k, None, wn, z)
    same = oracle.gate(x, wg, k, None, wn, z, route=g.topk_idx)
    for f in ("topk_idx", "topk_w", "importance", "load", "probs"):
        np.testing.assert_array_equal(getattr(same, f), getattr(g, f), err_msg=f)
    t = 5
    order = np.argsort(-g.H[t], kind="stable")
    route = g.topk_idx.copy()
    route[t, k - 1] = order[k]          # the (k+1)-th expert in place of the k-th
    h = oracle.gate(x, wg, k, None, wn, z, route=route)
    np.testing.assert_array_equal(h.topk_idx, route)
    vals = g.H[t, route[t]]
    np.testing.assert_allclose(h.topk_w[t], np.exp(vals - vals.max()) / np.exp(vals - vals.max()).sum(),
                               rtol=1e-14)
    assert h.importance.sum() == pytest.approx(T, rel=1e-14)
    other = np.setdiff1d(np.arange(n), [order[k - 1], order[k]])
    np.testing.assert_allclose(h.load[other], g.load[other], rtol=1e-14)
    assert not np.allclose(h.load[order[k - 1]], g.load[order[k - 1]], rtol=1e-9)
    # the two-level gate's own routing held fixed changes nothing
    a, b = 3, 4
    wg2, wn2 = r.standard_normal((a, b, d)), r.standard_normal((a, b, d))
    z1, z2 = r.standard_normal((T, a)), r.standard_normal((T, 2, b))
    gh = oracle.gate_hier(x, wg[:a], wn[:a], z1, 2, wg2, wn2, z2, 1)
    gh2 = oracle.gate_hier(x, wg[:a], wn[:a], z1, 2, wg2, wn2, z2, 1, route=gh["topk_idx"])
    for f in ("topk_idx", "topk_w", "importance", "load"):
        np.testing.assert_array_equal(gh2[f], gh[f], err_msg=f)
    assert gh2["zsum"] == gh["zsum"] and gh2["entsum"] == gh["entsum"]


def _two_level_golden():
    with open(os.path.join(GOLDEN, "two_level_layer.json")) as f:
        g = json.load(f)
    ns = {"L": math.log(2.0), "Phi": lambda z: float(ndtr(z)),
          "p": math.exp(0.5) / (1 + math.exp(0.5)), "q": 1 / (1 + math.exp(0.5))}

    def ev(v):
        if isinstance(v, list):
            return [ev(u) for u in v]
        if isinstance(v, str):
            return float(eval(v, {"__builtins__": {}}, ns))
        return v
    return g, ev


def two_level_golden_inputs():
    """The hand-worked two-level case of tests/golden/two_level_layer.json as
    arrays (noise weights and draws all zero)."""
    g, ev = _two_level_golden()
    inp = g["inputs"]
    T, d, a, b, k1 = inp["T"], inp["d"], inp["a"], inp["b"], inp["k1"]
    return dict(x=np.array(inp["x"], float), w_gate=np.array(inp["w_gate"], float),
                w_noise=np.zeros((a, d)), noise=np.zeros((T, a)),
                w_gate2=np.array(inp["w_gate2"], float), w_noise2=np.zeros((a, b, d)),
                noise2=np.zeros((T, k1, b)), k1=k1, k2=inp["k2"]), g, ev


def test_golden_two_level_load():
    """The two-level Importance and Load against the hand-worked case: four
    groups reached by 3, 2, 1 and 0 (token, slot) pairs, so Load_primary[g],
    |X_g| and T all differ and one group is empty.  Reading of [NOTES]
    "分层 MoE" with [PAPER] "負載平衡損失": Load_H[g*b+e] =
    Load_primary[g] * Load_g[e] / |X_g|, 0 for an unreached group."""
    inp, g, ev = two_level_golden_inputs()
    exp = g["expected"]
    out = oracle.gate_hier(inp["x"], inp["w_gate"], inp["w_noise"], inp["noise"], inp["k1"],
                           inp["w_gate2"], inp["w_noise2"], inp["noise2"], inp["k2"])
    pg = out["primary"]
    np.testing.assert_array_equal(pg.topk_idx, exp["primary_topk_idx"])
    np.testing.assert_allclose(pg.topk_w, ev(exp["primary_topk_w"]), rtol=1e-15)
    lp = np.array(ev(exp["load_primary"]))
    np.testing.assert_allclose(pg.load, lp, rtol=1e-14)
    np.testing.assert_array_equal(out["group_tokens"], exp["group_tokens"])
    ls = np.array(ev(exp["load_secondary"]))
    np.testing.assert_allclose(out["load_secondary"], ls, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(out["topk_idx"], exp["topk_idx"])
    np.testing.assert_allclose(out["topk_w"], ev(exp["topk_w"]), rtol=1e-15)
    np.testing.assert_allclose(out["importance"], ev(exp["importance"]), rtol=1e-15, atol=0)
    want = np.array(ev(exp["load"]))
    np.testing.assert_allclose(out["load"], want, rtol=1e-14, atol=0)
    assert np.all(out["load"][9:] == 0.0)  # the unreached group

    # The case separates the reading from its plausible misreadings: each of
    # these differs from the hand values by far more than the tolerance.
    a, b = ls.shape
    T = inp["x"].shape[0]
    gt = np.array(exp["group_tokens"], float)
    reached = gt > 0
    no_primary = np.where(reached[:, None], ls, 0.0).ravel()
    over_T = np.where(reached[:, None], lp[:, None] * ls / T, 0.0).ravel()
    counts_for_load = np.where(reached[:, None], gt[:, None] * ls / np.maximum(gt, 1)[:, None],
                               0.0).ravel()
    transposed = np.where(reached[:, None], lp[:, None] * ls / np.maximum(gt, 1)[:, None],
                          0.0).T.ravel()
    for wrong in (no_primary, over_T, counts_for_load, transposed):
        assert np.max(np.abs(wrong - want)) > 1e-3

    # The two-level loss is w_load * CV^2 over all a*b entries.
    losses = oracle.aux(T, 2, out["importance"], out["load"],
                        oracle.dispatch(out["topk_idx"], a * b)["counts_pre"], 0.1, 0.1, 1.0)
    cv2 = np.mean((want - want.mean()) ** 2) / want.mean() ** 2
    assert losses[1] == pytest.approx(0.1 * cv2, rel=1e-13)


def test_hierarchical_matches_dense_two_level_sum():
    # y = sum_g Gp(x)_g sum_e G_g(x)_e E_{g,e}(x), evaluated densely per token.
    r = rng(17)
    T, d, a, b, k1, k2, h = 9, 5, 3, 4, 2, 2, 6
    x = r.standard_normal((T, d))
    wg1, wn1 = r.standard_normal((a, d)), r.standard_normal((a, d))
    z1 = r.standard_normal((T, a))
    wg2, wn2 = r.standard_normal((a, b, d)), r.standard_normal((a, b, d))
    z2 = r.standard_normal((T, k1, b))
    w1 = r.standard_normal((a * b, h, d))
    w2 = r.standard_normal((a * b, d, h))
    out = oracle.forward_hier(x, wg1, wn1, z1, k1, wg2, wn2, z2, k2, w1, w2)
    y = np.zeros((T, d))
    imp = np.zeros(a * b)
    for t in range(T):
        Hp = x[t] @ wg1.T + z1[t] * np.logaddexp(0, x[t] @ wn1.T)
        order = sorted(range(a), key=lambda j: (-Hp[j], j))[:k1]
        wp = np.exp(Hp[order] - Hp[order[0]])
        wp /= wp.sum()
        for s, g in enumerate(order):
            Hs = x[t] @ wg2[g].T + z2[t, s] * np.logaddexp(0, x[t] @ wn2[g].T)
            o2 = sorted(range(b), key=lambda j: (-Hs[j], j))[:k2]
            ws = np.exp(Hs[o2] - Hs[o2[0]])
            ws /= ws.sum()
            for e, w in zip(o2, ws):
                y[t] += wp[s] * w * _ffn_np(x[t:t + 1], w1[g * b + e], w2[g * b + e])[0]
                imp[g * b + e] += wp[s] * w
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["gate"]["importance"], imp, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# FP8 E4M3 expert weights
# ---------------------------------------------------------------------------

def test_e4m3_decode_every_code_matches_torch():
    """All 256 codes against torch's float8_e4m3fn decoding (NaN at
    S.1111.111, signed zero, subnormals below 2^-6, largest 448)."""
    ours = oracle.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[0x7e] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_rounding():
    """Round to nearest even against torch's float -> float8_e4m3fn cast, on
    every code value, every midpoint between neighbours (the ties), points
    just off the midpoints and random values in [-448, 448]."""
    mags = oracle.e4m3_decode(np.arange(0x7f))
    mids = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                           np.random.default_rng(0).uniform(-448, 448, 4000)])
    vals = np.concatenate([vals, -vals]).astype(np.float32).astype(np.float64)
    ours = oracle.e4m3_encode(vals)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)
    # beyond the largest finite value the encoder saturates
    np.testing.assert_array_equal(oracle.e4m3_encode([460.0, -1e6]), [0x7e, 0xfe])


def test_fp8_row_quantization_closed_form_and_bound():
    """Row (1, -2, 0.5, 4): scale 4/448 in single precision, codes of 112,
    -224, 56, 448; a zero row gets scale 1 and zero codes.  On random rows
    every dequantized value is within half an E4M3 step of the weight:
    2^-4 relative for normals, 2^-10 * scale below 2^-6 * scale."""
    c, s = oracle.quantize_fp8_rows(np.array([[1, -2, 0.5, 4], [0, 0, 0, 0]], float))
    assert s[0] == float(np.float32(4.0) / np.float32(448.0)) and s[1] == 1.0
    np.testing.assert_array_equal(c[0], oracle.e4m3_encode([112, -224, 56, 448]))
    np.testing.assert_array_equal(c[1], 0)
    w = oracle.bf16_round(np.random.default_rng(1).standard_normal((16, 64)) * 0.05)
    c, s = oracle.quantize_fp8_rows(w)
    deq = oracle.dequantize_fp8_rows(c, s)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(deq - w) <= bound)
    assert np.allclose(np.max(np.abs(deq), axis=1), 448 * s, rtol=1e-6)


def test_fp8_expert_single_expert_numpy():
    """One expert with FP8 weights: the oracle FFN on the dequantized weights
    equals a numpy dense FFN over the same values (bf16 activations)."""
    rng = np.random.default_rng(6)
    T, d, h = 7, 64, 128
    x = rng.standard_normal((T, d))
    w1 = oracle.bf16_round(rng.standard_normal((h, d)) / 8)
    w2 = oracle.bf16_round(rng.standard_normal((d, h)) / 11)
    q1 = oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(w1))
    q2 = oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(w2))
    y = oracle.expert_ffn(x, q1, q2, bf16=True)
    hid = oracle.bf16_round(np.maximum(oracle.bf16_round(x) @ q1.T, 0))
    np.testing.assert_allclose(y, hid @ q2.T, rtol=1e-12, atol=1e-12)


def test_results_do_not_depend_on_thread_count():
    # The CPU baseline is timed on one core and on all cores; both runs must
    # compute the same numbers bit for bit (disjoint per-element outputs,
    # serial sums over tokens).
    r = rng(31)
    T, d, n, k, h = 300, 16, 12, 3, 8
    x = r.standard_normal((T, d))
    wg = r.standard_normal((n, d))
    wn = r.standard_normal((n, d))
    z = r.standard_normal((T, n))
    w1 = r.standard_normal((n, h, d))
    w2 = r.standard_normal((n, d, h))
    threads = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        one = oracle.forward(x, wg, k, w1, w2, w_noise=wn, noise=z, capacity_factor=1.0)
        oracle.set_num_threads(max(2, threads))
        many = oracle.forward(x, wg, k, w1, w2, w_noise=wn, noise=z, capacity_factor=1.0)
    finally:
        oracle.set_num_threads(threads)
    np.testing.assert_array_equal(one["y"], many["y"])
    np.testing.assert_array_equal(one["losses"], many["losses"])
    np.testing.assert_array_equal(one["gate"].topk_idx, many["gate"].topk_idx)
