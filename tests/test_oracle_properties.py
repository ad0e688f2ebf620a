"""Property-based pins of the oracle (hypothesis, CPU): random shapes from the
degenerate to the wide (T in [0, 300] tokens, n in [1, 300] experts, k in
[1, n]) with values drawn from a small quantised set, so ties and -0.0 / +0.0
pairs are common, each checked against a brute-force restatement of the
definitions:

* KeepTopK ([PAPER] Noisy Top-K gating): the kept set is the k largest H,
  lower index first among equal values (-0.0 equal to +0.0), the slots in
  descending H; H_(k), H_(k+1) the k-th and (k+1)-th largest values (-inf
  past n);
* kth_excluding(H, k, i) (the load estimator's threshold): the k-th largest of
  H with entry i deleted, by literally deleting it and sorting;
* the kept weights: a softmax over the kept values, summing to 1;
* dispatch ([NOTES] merged batches, [SURVEY] 3.2 capacity): the per-expert
  lists built pair by pair in (token, slot) order, first come first served.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle

VALUES = np.array([-3.0, -1.5, -1.0, -0.5, -0.0, 0.0, 0.25, 0.5, 1.0, 2.0, 7.5])


def _H(seed, T, n, spread):
    r = np.random.default_rng(seed)
    if spread:  # a mix of quantised values and continuous ones
        H = r.choice(VALUES, size=(T, n))
        cont = r.random((T, n)) < 0.5
        return np.where(cont, r.standard_normal((T, n)), H)
    return r.choice(VALUES, size=(T, n))


def _order(v):
    # descending value, lower index first; -0.0 == +0.0 since -(-0.0) == -(0.0)
    return sorted(range(len(v)), key=lambda j: (-v[j], j))


shapes = st.tuples(st.integers(0, 300), st.integers(1, 300), st.floats(0.0, 1.0),
                   st.integers(0, 2**31 - 1), st.booleans())


@settings(max_examples=60, deadline=None)
@given(shapes)
def test_keep_topk_matches_sorting(shape):
    T, n, kf, seed, spread = shape
    k = 1 + int(kf * (n - 1))
    H = _H(seed, T, n, spread)
    idx, hk, hk1 = oracle.keep_topk(H, k)
    assert idx.shape == (T, k)
    for t in range(T):
        o = _order(H[t])
        assert list(idx[t]) == o[:k]
        vals = sorted(H[t], reverse=True)
        assert hk[t] == vals[k - 1]
        assert hk1[t] == (vals[k] if k < n else -math.inf)


@settings(max_examples=40, deadline=None)
@given(shapes)
def test_load_threshold_is_kth_excluding(shape):
    T, n, kf, seed, spread = shape
    k = 1 + int(kf * (n - 1))
    T = min(T, 12)  # the brute force deletes every expert in turn
    H = _H(seed, T, n, spread)
    r = np.random.default_rng(seed + 1)
    clean = H - r.choice([0.0, 0.5, -0.25], size=H.shape)
    sp = r.choice([0.5, 1.0, 2.0], size=H.shape)
    idx, hk, hk1 = oracle.keep_topk(H, k)
    load, P = oracle.load(clean, sp, idx, hk, hk1)
    for t in range(T):
        for i in range(n):
            others = sorted(np.delete(H[t], i), reverse=True)
            thr = others[k - 1] if k - 1 < len(others) else -math.inf
            want = 1.0 if thr == -math.inf else oracle.phi((clean[t, i] - thr) / sp[t, i])
            assert P[t, i] == pytest.approx(want, rel=1e-14, abs=1e-300)
    np.testing.assert_allclose(load, P.sum(0) if T else np.zeros(n), rtol=1e-13, atol=0)


@settings(max_examples=40, deadline=None)
@given(shapes)
def test_kept_weights_are_a_softmax_of_the_kept_values(shape):
    T, n, kf, seed, spread = shape
    k = 1 + int(kf * (n - 1))
    H = _H(seed, T, n, spread)
    idx, _, _ = oracle.keep_topk(H, k)
    w, probs = oracle.gate_weights(H, idx)
    for t in range(T):
        v = H[t][idx[t]]
        e = np.exp(v - v.max())
        np.testing.assert_allclose(w[t], e / e.sum(), rtol=1e-13, atol=1e-300)
        assert w[t].sum() == pytest.approx(1.0, rel=1e-13)
        dense = np.zeros(n)
        dense[idx[t]] = w[t]
        np.testing.assert_array_equal(probs[t], dense)


@settings(max_examples=60, deadline=None)
@given(shapes, st.sampled_from([0.0, 0.3, 1.0, 1.25, 4.0]))
def test_dispatch_matches_pair_by_pair_lists(shape, cf):
    T, n, kf, seed, _ = shape
    k = 1 + int(kf * (min(n, 64) - 1))
    r = np.random.default_rng(seed)
    # skewed picks: experts repeat across tokens, never within a token
    p = np.linspace(1.0, 3.0, n) ** 3
    idx = np.array([r.choice(n, k, replace=False, p=p / p.sum()) for _ in range(T)],
                   dtype=np.int32).reshape(T, k)
    d = oracle.dispatch(idx, n, cf)
    cap = math.floor(cf * T * k / n) if cf > 0 else T * k + 1
    lists = [[] for _ in range(n)]
    slot = -np.ones((T, k), np.int64)
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            if len(lists[e]) < cap:
                lists[e].append(t)
                slot[t, s] = len(lists[e]) - 1  # position within e, fixed to a row below
    counts = np.array([len(l) for l in lists])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rows = np.where(slot >= 0, offsets[np.where(slot >= 0, idx, 0)] + slot, -1)
    np.testing.assert_array_equal(d["counts_pre"], np.bincount(idx.reshape(-1), minlength=n))
    np.testing.assert_array_equal(d["counts"], counts)
    np.testing.assert_array_equal(d["offsets"], offsets)
    np.testing.assert_array_equal(d["perm"], [t for l in lists for t in l])
    np.testing.assert_array_equal(d["slot_pos"], rows)
