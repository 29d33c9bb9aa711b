"""Pins of the routing / permutation oracle (oracle/route.py).

* top-k indices against an independent brute force (np.lexsort with the tie rule),
  on logits with forced ties and signed zeros;
* probabilities: sum to 1, k = 1 gives 1, and they equal the full softmax over all
  E logits renormalised over the selected k (a different formula, same value);
* split_sizes equal np.bincount and sum to T*k; offsets are multiples of ALIGN;
* permutation: a bijection on assignments, rows increase within a group, padding is
  -1, and for ALIGN = 1 it equals np.argsort(expert_of_assignment, kind="stable");
* router backward: central differences of the oracle's own forward routing (selection
  held fixed), of softmax(l[idx]) with a repeated index, and the invariants (rows sum
  to 0, zeros off the selection, k = 1 and a constant d_prob give 0).
"""
import numpy as np
import pytest

import synth
from oracle import route as rt


def brute_topk(l, k):
    T, E = l.shape
    out = np.zeros((T, k), np.int32)
    for t in range(T):
        # lexsort sorts by the last key first: primary key -logit, secondary index
        order = np.lexsort((np.arange(E), -l[t]))
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("E,k", [(4, 2), (8, 2), (8, 1), (5, 5), (16, 4)])
def test_topk_matches_bruteforce_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    l = np.round(rng.standard_normal((300, E)) * 2) / 2   # many exact ties
    l = l.astype(np.float32)
    l[::7] = 0.0
    l[1::7, 0] = -0.0
    idx, p = rt.route(l, k)
    np.testing.assert_array_equal(idx, brute_topk(l.astype(np.float64), k))
    for t in range(l.shape[0]):
        assert len(set(idx[t])) == k
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=4 * np.finfo(float).eps)
    assert np.all(np.diff(p, axis=1) <= 0)   # slot order follows the logit order


def test_ties_go_to_lower_index():
    l = np.array([[1.0, 3.0, 3.0, 3.0], [0.0, -0.0, 0.0, -1.0]], np.float32)
    idx, p = rt.route(l, 2)
    np.testing.assert_array_equal(idx, [[1, 2], [0, 1]])
    np.testing.assert_allclose(p, 0.5)


def test_prob_equals_renormalised_full_softmax():
    w = synth.WORKLOADS[0]
    l = synth.logits(w).astype(np.float64)
    idx, p = rt.route(l, w.k)
    full = np.exp(l - l.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(p, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)


def test_k1_prob_is_one():
    l = np.random.default_rng(1).standard_normal((50, 6)).astype(np.float32)
    idx, p = rt.route(l, 1)
    assert np.all(p == 1.0)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(l, axis=1))


@pytest.mark.parametrize("align", [1, 32, 8])
def test_split_sizes_offsets_permutation(align):
    w = synth.WORKLOADS[0]
    l = synth.logits(w)
    idx, p = rt.route(l, w.k)
    s = rt.split_sizes(idx, w.E)
    np.testing.assert_array_equal(s, np.bincount(idx.ravel(), minlength=w.E))
    assert s.sum() == w.T * w.k
    off = rt.group_offsets(s, align)
    assert off[0] == 0 and np.all(off % align == 0) and np.all(np.diff(off) >= s)
    src, pos = rt.perm_rows(w.T, w.k, w.E, align), None
    perm_src, perm_pos = rt.permutation(idx, w.E, align)
    assert len(perm_src) == src and src % 32 == 0 and off[-1] <= src
    # bijection between assignments and non-padding rows
    for t in range(w.T):
        for i in range(w.k):
            assert perm_src[perm_pos[t, i]] == t
    assert np.count_nonzero(perm_src >= 0) == w.T * w.k
    for e in range(w.E):
        rows = perm_pos[idx == e]
        assert np.all((rows >= off[e]) & (rows < off[e] + s[e]))
        assert np.all(perm_src[off[e] + s[e]: off[e + 1]] == -1)
        # stable: rows increase with (t, i) order
        tt, ii = np.nonzero(idx == e)
        order = np.lexsort((ii, tt))
        assert np.all(np.diff(perm_pos[tt[order], ii[order]]) == 1)
    if align == 1:
        flat_e = idx.ravel()
        order = np.argsort(flat_e, kind="stable")
        np.testing.assert_array_equal(perm_src[: w.T * w.k], order // w.k)


def test_empty_experts_and_single_expert():
    idx = np.array([[2, 0], [2, 0], [0, 2]], np.int32)
    perm_src, perm_pos = rt.permutation(idx, 4, 32)
    s = rt.split_sizes(idx, 4)
    np.testing.assert_array_equal(s, [3, 0, 3, 0])
    np.testing.assert_array_equal(rt.group_offsets(s, 32), [0, 32, 32, 64, 64])
    np.testing.assert_array_equal(perm_pos, [[32, 0], [33, 1], [2, 34]])


def test_permutation_with_repeated_experts_in_a_token():
    """Caller-given indices may name one expert in several slots of a token: every slot
    still gets its own row, in (t, i) order.  Pinned by the stable argsort special case
    (align 1) and by hand on a small case."""
    idx = np.array([[1, 1], [0, 1], [1, 0], [0, 0]], np.int32)
    perm_src, perm_pos = rt.permutation(idx, 2, 1)
    np.testing.assert_array_equal(rt.split_sizes(idx, 2), [4, 4])
    # expert 0: (1,0) (2,1) (3,0) (3,1); expert 1: (0,0) (0,1) (1,1) (2,0)
    np.testing.assert_array_equal(perm_pos, [[4, 5], [0, 6], [7, 1], [2, 3]])
    np.testing.assert_array_equal(perm_src[:8], [1, 2, 3, 3, 0, 0, 1, 2])
    rng = np.random.default_rng(5)
    for E, k in ((3, 4), (6, 2), (1, 3)):
        idx = rng.integers(0, E, size=(200, k)).astype(np.int32)
        perm_src, perm_pos = rt.permutation(idx, E, 1)
        order = np.argsort(idx.ravel(), kind="stable")
        np.testing.assert_array_equal(perm_src[: idx.size], order // k)
        np.testing.assert_array_equal(perm_pos.ravel()[order], np.arange(idx.size))


def test_prob_permuted():
    idx = np.array([[1, 0], [0, 1]], np.int32)
    p = np.array([[0.7, 0.3], [0.6, 0.4]])
    perm_src, perm_pos = rt.permutation(idx, 2, 1)
    pp = rt.prob_permuted(p, perm_pos, len(perm_src))
    np.testing.assert_allclose(pp[:4], [0.3, 0.6, 0.7, 0.4])


# ---------------------------------------------------------------- router backward
def _fd_token(fwd, l_row, dp_row, h):
    """Central differences of L(l) = <fwd(l), dp> for one token, one logit at a time."""
    g = np.zeros_like(l_row)
    for e in range(l_row.shape[0]):
        lp, lm = l_row.copy(), l_row.copy()
        lp[e] += h
        lm[e] -= h
        g[e] = (np.dot(fwd(lp), dp_row) - np.dot(fwd(lm), dp_row)) / (2 * h)
    return g


@pytest.mark.parametrize("E,k", [(8, 2), (8, 4), (16, 3), (4, 4)])
def test_router_bwd_matches_finite_differences_of_route(E, k):
    """d_logits against numerical derivatives of the oracle's own forward routing:
    the selection and slot order stay fixed under the perturbation (all logits of a
    token are kept > 1e-3 apart, far above the step)."""
    rng = np.random.default_rng(100 + E * k)
    T, h = 24, 1e-6
    l = rng.standard_normal((T, E))
    for t in range(T):
        while np.min(np.diff(np.sort(l[t]))) < 1e-3:
            l[t] = rng.standard_normal(E)
    idx, p = rt.route(l, k)
    dp = rng.standard_normal((T, k))
    got = rt.router_bwd(idx, p, dp, E)
    for t in range(T):
        sel = idx[t].copy()
        fwd = lambda lr: rt.route(lr[None, :], k)[1][0]
        g = _fd_token(fwd, l[t], dp[t], h)
        np.testing.assert_array_equal(rt.route(l[t][None, :], k)[0][0], sel)
        np.testing.assert_allclose(got[t], g, rtol=0, atol=1e-7)


def test_router_bwd_duplicate_slots_sum():
    """Two slots gathering the same logit: the gradient is the sum over both, as the
    numerical derivative of softmax(l[idx]) (a forward written here) shows."""
    rng = np.random.default_rng(7)
    E, T = 6, 10
    l = rng.standard_normal((T, E))
    idx = np.array([[2, 2, 5], [0, 1, 0]] * 5, np.int32)

    def fwd_for(t):
        def f(lr):
            z = lr[idx[t]]
            ez = np.exp(z - z.max())
            return ez / ez.sum()
        return f

    p = np.stack([fwd_for(t)(l[t]) for t in range(T)])
    dp = rng.standard_normal((T, 3))
    got = rt.router_bwd(idx, p, dp, E)
    for t in range(T):
        np.testing.assert_allclose(got[t], _fd_token(fwd_for(t), l[t], dp[t], 1e-6), rtol=0, atol=1e-7)


def test_router_bwd_invariants():
    """Shift invariance of the softmax (each row sums to 0), zeros off the selection,
    k = 1 and a constant d_prob give no gradient."""
    rng = np.random.default_rng(3)
    T, E, k = 40, 8, 3
    l = rng.standard_normal((T, E))
    idx, p = rt.route(l, k)
    dp = rng.standard_normal((T, k))
    g = rt.router_bwd(idx, p, dp, E)
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-15)
    for t in range(T):
        off = np.setdiff1d(np.arange(E), idx[t])
        assert np.all(g[t, off] == 0.0)
    i1, p1 = rt.route(l, 1)
    assert np.all(rt.router_bwd(i1, p1, rng.standard_normal((T, 1)), E) == 0.0)
    assert np.abs(rt.router_bwd(idx, p, np.full((T, k), 0.37), E)).max() < 1e-16
