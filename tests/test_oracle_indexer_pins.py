"""Pins of the lightning-indexer oracle (oracle/indexer.py).

Source: "Ch 04 · CSA — 长上下文的快通道", section 4: the index score of
query t and key s is the w-weighted sum over the indexer heads of
ReLU(q_{t,h} . K_s); query t keeps the entries of its k largest scores.

Each check below is a fact fixed by that definition and by plain arithmetic,
not by the oracle's own code: hand-worked values, the identity
ReLU(x) - ReLU(-x) = x (which turns the score difference of Q and -Q into one
matrix product), sign and scaling laws, a pure-Python triple loop, and for the
selection an exhaustive search over all k-subsets.  The planted-mistake tests
show that a dropped ReLU, dropped head weights, a reversed tie-break and an
off-by-one visibility mask each fail one of these checks.
"""

import itertools

import numpy as np
import pytest

import oracle


def _data(T=3, H=5, c=7, N=11, seed=0):
    rng = np.random.default_rng([seed, 99])
    return rng.normal(size=(T, H, c)), rng.normal(size=(T, H)), rng.normal(size=(N, c))


# ------------------------------------------------------------------ scores

def test_hand_values():
    # One query, two heads of 2 dims, three keys, worked by hand:
    #   head 1: q = (1, 2),  dots with K = (1,0), (0,1), (-1,-1): 1, 2, -3 -> ReLU 1, 2, 0
    #   head 2: q = (-1, 1), dots: -1, 1, 0                            -> ReLU 0, 1, 0
    #   weights (0.5, 2): I = (0.5*1 + 2*0, 0.5*2 + 2*1, 0) = (0.5, 3, 0)
    Q = np.array([[[1.0, 2.0], [-1.0, 1.0]]])
    w = np.array([[0.5, 2.0]])
    K = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, -1.0]])
    np.testing.assert_array_equal(oracle.index_scores(Q, w, K), [[0.5, 3.0, 0.0]])
    idx, val = oracle.top_k(oracle.index_scores(Q, w, K), 2)
    np.testing.assert_array_equal(idx, [[0, 1]])
    np.testing.assert_array_equal(val, [[0.5, 3.0]])


def _check_relu_identity(score_fn):
    # ReLU(x) - ReLU(-x) = x, so I(Q) - I(-Q) = sum_h w_h (q_h . K): one matmul per head
    Q, w, K = _data()
    lhs = score_fn(Q, w, K) - score_fn(-Q, w, K)
    rhs = np.stack([sum(w[t, h] * (K @ Q[t, h]) for h in range(Q.shape[1])) for t in range(Q.shape[0])])
    return np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_relu_difference_identity():
    assert _check_relu_identity(oracle.index_scores)


def test_negative_dots_score_zero_for_any_weights():
    Q, w, K = _data()
    I = oracle.index_scores(np.abs(Q), w * 100.0, -np.abs(K))   # every dot product <= 0
    np.testing.assert_array_equal(I, np.zeros_like(I))


def test_single_head_nonnegative_is_a_matrix_product():
    Q, _, K = _data(H=1)
    Q, K = np.abs(Q), np.abs(K)
    I = oracle.index_scores(Q, np.ones((Q.shape[0], 1)), K)
    np.testing.assert_allclose(I, Q[:, 0, :] @ K.T, rtol=1e-14)


def test_scaling_laws():
    Q, w, K = _data()
    I = oracle.index_scores(Q, w, K)
    np.testing.assert_allclose(oracle.index_scores(2.5 * Q, w, K), 2.5 * I, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.index_scores(Q, -3.0 * w, K), -3.0 * I, rtol=1e-13, atol=1e-13)
    # heads are independent: the score with all heads is the sum of one-head scores
    parts = sum(oracle.index_scores(Q[:, h:h + 1], w[:, h:h + 1], K) for h in range(Q.shape[1]))
    np.testing.assert_allclose(parts, I, rtol=1e-13, atol=1e-13)


def _loop_scores(Q, w, K):
    T, H, c = Q.shape
    out = np.zeros((T, K.shape[0]))
    for t in range(T):
        for s in range(K.shape[0]):
            tot = 0.0
            for h in range(H):
                dot = 0.0
                for i in range(c):
                    dot += Q[t, h, i] * K[s, i]
                tot += w[t, h] * max(dot, 0.0)
            out[t, s] = tot
    return out


def test_brute_force_loops():
    Q, w, K = _data(T=2, H=4, c=5, N=6, seed=3)
    np.testing.assert_allclose(oracle.index_scores(Q, w, K), _loop_scores(Q, w, K), rtol=1e-12, atol=1e-12)


def test_visibility_mask():
    Q, w, K = _data()
    nv = np.array([0, 4, 11])
    I = oracle.index_scores(Q, w, K, n_valid=nv)
    full = oracle.index_scores(Q, w, K)
    assert np.all(I[0] == -np.inf)
    np.testing.assert_array_equal(I[1, :4], full[1, :4])
    assert np.all(I[1, 4:] == -np.inf)
    np.testing.assert_array_equal(I[2], full[2])


# --------------------------------------------------------------- selection

def _exhaustive_top_k(row, k):
    """The unique visible k-subset every member of which outranks every
    visible non-member under (higher score, then smaller index)."""
    vis = [s for s in range(len(row)) if row[s] > -np.inf]
    if len(vis) <= k:
        return sorted(vis)
    better = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    found = [S for S in itertools.combinations(vis, k)
             if all(better(a, b) for a in S for b in vis if b not in S)]
    assert len(found) == 1
    return list(found[0])


def test_top_k_matches_exhaustive_search():
    rng = np.random.default_rng([5, 1])
    for trial in range(40):
        N = int(rng.integers(1, 9))
        row = rng.integers(-2, 3, size=N).astype(np.float64)   # small integers: many ties
        nv = int(rng.integers(0, N + 1))
        row[nv:] = -np.inf
        k = int(rng.integers(1, 6))
        idx, val = oracle.top_k(row[None, :], k)
        want = _exhaustive_top_k(row, k)
        assert list(idx[0, :len(want)]) == want, (row, k)
        assert np.all(idx[0, len(want):] == -1) and np.all(val[0, len(want):] == -np.inf)
        np.testing.assert_array_equal(val[0, :len(want)], row[want])


def test_top_k_ties_and_stable_argsort():
    idx, _ = oracle.top_k(np.array([[2.0, 5.0, 2.0, 5.0, 1.0]]), 3)
    np.testing.assert_array_equal(idx, [[0, 1, 3]])        # the tie at 2 goes to index 0
    rng = np.random.default_rng([5, 2])
    I = rng.normal(size=(4, 300))
    idx, _ = oracle.top_k(I, 17)
    ref = np.sort(np.argsort(-I, axis=1, kind="stable")[:, :17], axis=1)
    np.testing.assert_array_equal(idx, ref)


# --------------------------------------------------------- planted mistakes

def test_planted_score_mistakes_are_caught():
    no_relu = lambda Q, w, K: np.einsum("th,thc,sc->ts", w, Q, K)
    no_weight = lambda Q, w, K: oracle.index_scores(Q, np.ones_like(w), K)
    assert not _check_relu_identity(no_relu)
    assert not _check_relu_identity(no_weight)
    Q, w, K = _data()
    assert not np.allclose(no_relu(Q, w, K), _loop_scores(Q, w, K))
    assert not np.allclose(no_weight(Q, w, K), _loop_scores(Q, w, K))
    # a max(dot, 0) taken after the head weight (ReLU(w * dot)) breaks the sign law
    late_relu = lambda Q, w, K: np.maximum(np.einsum("th,thc,sc->ths", w, Q, K), 0).sum(1)
    assert not np.allclose(late_relu(Q, -3.0 * w, K), -3.0 * late_relu(Q, w, K))


@pytest.mark.parametrize("mutant", ["reversed_ties", "mask_off_by_one"])
def test_planted_selection_mistakes_are_caught(mutant):
    def bad(row, k):
        vis = [s for s in range(len(row)) if row[s] > -np.inf]
        if mutant == "mask_off_by_one":
            vis = vis + [len(vis)] if len(vis) < len(row) else vis
        key = (lambda s: (-row[s], -s)) if mutant == "reversed_ties" else (lambda s: (-row[s], s))
        return sorted(sorted(vis, key=key)[:k])

    rng = np.random.default_rng([5, 3])
    caught = False
    for _ in range(40):
        N = int(rng.integers(2, 9))
        row = rng.integers(-2, 3, size=N).astype(np.float64)
        row[int(rng.integers(0, N)):] = -np.inf
        k = int(rng.integers(1, 5))
        caught |= bad(row, k) != _exhaustive_top_k(row, k)
    assert caught
