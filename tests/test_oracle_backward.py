"""Pins of the oracle's backward pass (CPU only).

The backward is pinned to the oracle's forward, which has its own pins, by
central finite differences of the scalar objective
L = sum <dy, y> + sum dl * losses, at fp64 and fp32 experts (no bf16
rounding, so L is smooth wherever the selection, the capacity drops and the
ReLU pattern do not change).  Each case checks a random sample of entries of
every input and parameter tensor.  A plausible slip anywhere in the gate's
chain (a dropped term of the load estimator's threshold, a sign, the softmax
centring, the z-loss factor) moves some sampled entry by far more than the
tolerance; mistakes in the expert part show in every weight gradient.
"""
import numpy as np
import pytest

import oracle as O

EPS = 1e-6
TOL = 1e-6  # |fd - analytic| <= TOL * (1 + |analytic|); the FD error is ~1e-9 here


def _problem(seed, mode, act, noisy, shared, n=6, T=40, d=12, h=10, bias=True):
    rng = np.random.default_rng(seed)
    P = dict(x=rng.standard_normal((T, d)), w_gate=rng.standard_normal((n, d)) * 0.5,
             w1=rng.standard_normal((n, h, d)) / np.sqrt(d),
             w2=rng.standard_normal((n, d, h)) / np.sqrt(h))
    if bias:
        P["b_gate"] = rng.standard_normal(n) * 0.3
    if noisy:
        P["w_noise"] = rng.standard_normal((n, d)) * 0.3
    if act == O.ACT_SWIGLU:
        P["w3"] = rng.standard_normal((n, h, d)) / np.sqrt(d)
    else:
        P["b1"] = rng.standard_normal((n, h)) * 0.1
        P["b2"] = rng.standard_normal((n, d)) * 0.1
    if shared:
        P["ws1"] = rng.standard_normal((h, d)) / np.sqrt(d)
        P["ws2"] = rng.standard_normal((d, h)) / np.sqrt(h)
        if act == O.ACT_SWIGLU:
            P["ws3"] = rng.standard_normal((h, d)) / np.sqrt(d)
    noise = rng.standard_normal((T, n)) if noisy else None
    dy = rng.standard_normal((T, d))
    dl = rng.standard_normal(5)
    return rng, P, noise, dy, dl


_GRAD = dict(x="dx", w_gate="dw_gate", b_gate="db_gate", w_noise="dw_noise", w1="dw1",
             b1="db1", w3="dw3", w2="dw2", b2="db2", ws1="dws1", ws3="dws3", ws2="dws2")
_OPT = ("b_gate", "w_noise", "b1", "w3", "b2", "ws1", "ws3", "ws2")


def _kwargs(P, noise, mode, act, cf):
    kw = dict(noise=noise, mode=mode, act=act, capacity_factor=cf, w_importance=0.3,
              w_load=0.4, alpha=0.5, w_z=0.2, w_entropy=0.7)
    for name in _OPT:
        kw[name] = P.get(name)
    return kw


def _objective(P, k, noise, mode, act, cf, dy, dl):
    f = O.forward(P["x"], P["w_gate"], k, P["w1"], P["w2"], **_kwargs(P, noise, mode, act, cf))
    return float((dy * f["y"]).sum() + (dl * f["losses"]).sum()), f


CASES = [
    # id, mode, act, noisy, capacity factor, shared expert, k
    ("noisy_topk2_relu", O.GATE_TOPK_SOFTMAX, O.ACT_RELU, True, 0.0, False, 2),
    ("noisy_topk2_capacity_shared", O.GATE_TOPK_SOFTMAX, O.ACT_RELU, True, 0.8, True, 2),
    ("switch_noisy_capacity", O.GATE_SWITCH_TOP1, O.ACT_RELU, True, 1.2, False, 1),
    ("switch_clean", O.GATE_SWITCH_TOP1, O.ACT_RELU, False, 0.0, False, 1),
    ("sigmoid_swiglu_shared", O.GATE_SIGMOID_BIAS, O.ACT_SWIGLU, False, 0.0, True, 3),
    ("topk_all_swiglu", O.GATE_TOPK_SOFTMAX, O.ACT_SWIGLU, False, 0.0, False, 6),
    ("noisy_topk_all", O.GATE_TOPK_SOFTMAX, O.ACT_RELU, True, 0.0, False, 6),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_finite_differences(case):
    _, mode, act, noisy, cf, shared, k = case
    rng, P, noise, dy, dl = _problem(7, mode, act, noisy, shared)
    _, f0 = _objective(P, k, noise, mode, act, cf, dy, dl)
    assert not f0["gate"].near_tie.any()
    g = O.backward(P["x"], P["w_gate"], k, P["w1"], P["w2"], dy, dl,
                   **_kwargs(P, noise, mode, act, cf))
    if cf > 0:
        assert (f0["dispatch"]["slot_pos"] < 0).any(), "the case should drop slots"
    for name, v in P.items():
        an = g[_GRAD[name]]
        if name == "b_gate" and mode == O.GATE_SIGMOID_BIAS:
            assert an is None  # the selection-only bias receives no gradient
            continue
        assert an.shape == v.shape
        for fi in rng.choice(v.size, size=min(8, v.size), replace=False):
            Pp = {a: b.copy() for a, b in P.items()}
            Pm = {a: b.copy() for a, b in P.items()}
            Pp[name].flat[fi] += EPS
            Pm[name].flat[fi] -= EPS
            lp, fp = _objective(Pp, k, noise, mode, act, cf, dy, dl)
            lm, fm = _objective(Pm, k, noise, mode, act, cf, dy, dl)
            # the perturbation must not change the discrete routing
            assert (fp["gate"].topk_idx == f0["gate"].topk_idx).all()
            assert (fm["gate"].topk_idx == f0["gate"].topk_idx).all()
            fd = (lp - lm) / (2 * EPS)
            assert abs(fd - an.flat[fi]) <= TOL * (1 + abs(an.flat[fi])), (name, fi, fd,
                                                                           an.flat[fi])


def test_cv2_grad_closed_form():
    # v = (1, 3): mean 2, var 1, CV^2 = 1/4; d/dv = (2/(n m^2)) ((v - m) - var/m)
    # = (1/4) * ((-1, 1) - 1/2) = (-3/8, 1/8)
    np.testing.assert_allclose(O.cv2_grad([1.0, 3.0]), [-0.375, 0.125], rtol=0, atol=1e-15)
    # scaling every entry leaves CV^2 unchanged: the gradient is orthogonal to v
    v = np.array([0.5, 2.0, 4.0, 1.5])
    assert abs(O.cv2_grad(v) @ v) < 1e-14
    # mean 0: CV^2 is defined as 0 and so is its gradient
    assert not O.cv2_grad([1.0, -1.0]).any()


def test_zero_upstream_gives_zero_gradients():
    rng, P, noise, dy, dl = _problem(3, O.GATE_TOPK_SOFTMAX, O.ACT_RELU, True, True)
    g = O.backward(P["x"], P["w_gate"], 2, P["w1"], P["w2"], np.zeros_like(dy), np.zeros(5),
                   **_kwargs(P, noise, O.GATE_TOPK_SOFTMAX, O.ACT_RELU, 0.0))
    for name in P:
        assert not g[_GRAD[name]].any(), name


def test_dropped_slots_carry_no_expert_gradient():
    # with capacity 0 < C every slot past C is dropped: an expert none of whose
    # rows survive gets zero weight gradients; with cf tiny every expert has C = 0
    rng, P, noise, dy, dl = _problem(5, O.GATE_TOPK_SOFTMAX, O.ACT_RELU, True, False)
    g = O.backward(P["x"], P["w_gate"], 2, P["w1"], P["w2"], dy, dl,
                   **_kwargs(P, noise, O.GATE_TOPK_SOFTMAX, O.ACT_RELU, 1e-3))
    assert (g["fwd"]["dispatch"]["slot_pos"] < 0).all()
    for name in ("dw1", "db1", "dw2", "db2"):
        assert not g[name].any(), name
    assert not g["dG"].any()


@pytest.mark.parametrize("noisy", [True, False], ids=["noisy", "clean"])
def test_two_level_backward_matches_finite_differences(noisy):
    """The two-level layer: product weights, the factorised load and both
    levels' gates, pinned by finite differences of forward_hier."""
    rng = np.random.default_rng(11)
    T, d, a, b, k1, k2, h = 36, 10, 3, 4, 2, 2, 8
    P = dict(x=rng.standard_normal((T, d)), w_gate=rng.standard_normal((a, d)) * 0.5,
             w_gate2=rng.standard_normal((a, b, d)) * 0.5,
             w1=rng.standard_normal((a * b, h, d)) / np.sqrt(d),
             w2=rng.standard_normal((a * b, d, h)) / np.sqrt(h),
             b1=rng.standard_normal((a * b, h)) * 0.1, b2=rng.standard_normal((a * b, d)) * 0.1)
    if noisy:
        P["w_noise"] = rng.standard_normal((a, d)) * 0.3
        P["w_noise2"] = rng.standard_normal((a, b, d)) * 0.3
    noise = rng.standard_normal((T, a)) if noisy else None
    noise2 = rng.standard_normal((T, k1, b)) if noisy else None
    dy = rng.standard_normal((T, d))
    dl = rng.standard_normal(5)
    kw = dict(w_importance=0.3, w_load=0.4, alpha=0.5, w_z=0.2, w_entropy=0.7)

    def objective(P):
        f = O.forward_hier(P["x"], P["w_gate"], P.get("w_noise"), noise, k1, P["w_gate2"],
                           P.get("w_noise2"), noise2, k2, P["w1"], P["w2"], b1=P["b1"],
                           b2=P["b2"], **kw)
        return float((dy * f["y"]).sum() + (dl * f["losses"]).sum()), f

    _, f0 = objective(P)
    assert not f0["gate"]["near_tie"].any()
    g = O.backward_hier(P["x"], P["w_gate"], P.get("w_noise"), noise, k1, P["w_gate2"],
                        P.get("w_noise2"), noise2, k2, P["w1"], P["w2"], dy, dl, b1=P["b1"],
                        b2=P["b2"], **kw)
    names = dict(x="dx", w_gate="dw_gate", w_noise="dw_noise", w_gate2="dw_gate2",
                 w_noise2="dw_noise2", w1="dw1", w2="dw2", b1="db1", b2="db2")
    for name, v in P.items():
        an = g[names[name]]
        assert an.shape == v.shape
        for fi in rng.choice(v.size, size=min(8, v.size), replace=False):
            Pp = {q: r.copy() for q, r in P.items()}
            Pm = {q: r.copy() for q, r in P.items()}
            Pp[name].flat[fi] += EPS
            Pm[name].flat[fi] -= EPS
            lp, fp = objective(Pp)
            lm, fm = objective(Pm)
            assert (fp["gate"]["topk_idx"] == f0["gate"]["topk_idx"]).all()
            assert (fm["gate"]["topk_idx"] == f0["gate"]["topk_idx"]).all()
            fd = (lp - lm) / (2 * EPS)
            assert abs(fd - an.flat[fi]) <= TOL * (1 + abs(an.flat[fi])), (name, fi, fd,
                                                                           an.flat[fi])
