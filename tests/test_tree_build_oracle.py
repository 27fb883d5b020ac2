"""Pins of the best-first tree-builder oracle against facts that do not come
from the oracle itself: brute-force enumeration of every path, closed forms for
chains, stars and tied scores, and float32 accumulation."""
import itertools

import numpy as np
import pytest

from oracle.tree_build_oracle import best_first_tree


def _unique_tokens(B, D, K):
    # token = 1000 * depth + candidate: a token names its (depth, candidate).
    t = np.zeros((B, D, K), dtype=np.int64)
    for d in range(D):
        t[:, d, :] = 1000 * (d + 1) + np.arange(K)
    return t


def _paths(parent, token, n):
    """Candidate path of each node 1..n, from the unique tokens."""
    out = []
    for i in range(1, n + 1):
        p, node = [], i
        while node > 0:
            p.append(int(token[node]) % 1000)
            node = int(parent[node])
        out.append(tuple(reversed(p)))
    return out


@pytest.mark.parametrize("K,D,budget,seed", [(3, 3, 12, 0), (2, 4, 20, 1), (4, 2, 19, 2), (3, 3, 39, 3),
                                             (5, 3, 31, 4)])
def test_matches_brute_force_top_n(K, D, budget, seed):
    """Strictly negative, untied log-probs: an ancestor always outscores its
    descendants, so best-first takes exactly the budget best paths of all
    K + K^2 + ... + K^D, in descending score (enumerated by brute force)."""
    rng = np.random.default_rng(seed)
    B = 3
    lp = -rng.uniform(0.05, 3.0, size=(B, D, K)).astype(np.float32)
    tok = _unique_tokens(B, D, K)
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(B, np.int64), budget)
    for b in range(B):
        allp = []
        for d in range(1, D + 1):
            for path in itertools.product(range(K), repeat=d):
                s = np.float64(0.0)
                for i, c in enumerate(path):
                    s += np.float64(lp[b, i, c])
                allp.append((-s, path))
        allp.sort()
        want = [p for _, p in allp[:budget]]
        assert n[b] == min(budget, len(allp))
        assert _paths(parent[b], token[b], int(n[b])) == want


@pytest.mark.parametrize("K,budget", [(1, 5), (2, 14), (3, 20), (4, 40)])
@pytest.mark.parametrize("value", [0.0, -1.0])
def test_tied_scores_give_breadth_first_order(K, budget, value):
    """Every log-prob equal: depth decides, then the parent index, then the
    candidate: the breadth-first numbering of the complete K-ary tree,
    parent(i) = (i - 1) // K, candidate (i - 1) % K, depth = level."""
    D = 8
    B = 2
    lp = np.full((B, D, K), value, dtype=np.float32)
    tok = _unique_tokens(B, D, K)
    parent, token, depth, score, n = best_first_tree(lp, tok, np.array([7, 9]), budget)
    cap = sum(K ** d for d in range(1, D + 1))
    assert (n == min(budget, cap)).all()
    for i in range(1, int(n[0]) + 1):
        want_par = (i - 1) // K
        assert parent[0, i] == want_par and parent[1, i] == want_par
        assert token[0, i] % 1000 == (i - 1) % K
        assert depth[0, i] == depth[0, want_par] + 1
        assert score[0, i] == np.float32(value) * depth[0, i]
    assert token[0, 0] == 7 and token[1, 0] == 9 and parent[0, 0] == -1 and score[0, 0] == 0.0


@pytest.mark.parametrize("D,budget", [(5, 3), (5, 5), (4, 9)])
def test_single_candidate_gives_a_chain(D, budget):
    rng = np.random.default_rng(5)
    lp = rng.normal(size=(2, D, 1)).astype(np.float32)
    tok = rng.integers(0, 50000, size=(2, D, 1))
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(2, np.int64), budget)
    m = min(D, budget)
    assert (n == m).all()
    for i in range(1, m + 1):
        assert (parent[:, i] == i - 1).all() and (depth[:, i] == i).all()
        assert (token[:, i] == tok[:, i - 1, 0]).all()
    assert (parent[:, m + 1:] == -1).all() and (token[:, m + 1:] == -1).all()
    assert (depth[:, m + 1:] == -1).all() and np.isneginf(score[:, m + 1:]).all()


def test_depth_one_gives_a_sorted_star():
    """D = 1: the root's children by descending log-prob, equal ones by
    candidate index: a stable sort."""
    rng = np.random.default_rng(6)
    K = 16
    lp = rng.integers(-4, 1, size=(3, 1, K)).astype(np.float32)  # many ties
    tok = rng.integers(0, 1000, size=(3, 1, K))
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(3, np.int64), 10)
    for b in range(3):
        order = np.argsort(-lp[b, 0], kind="stable")[:10]
        assert (token[b, 1:11] == tok[b, 0, order]).all()
        assert (parent[b, 1:11] == 0).all()
        assert (score[b, 1:11] == lp[b, 0, order]).all()


def test_nan_counts_as_minus_infinity():
    lp = np.array([[[np.nan, -1.0, -np.inf, -2.0]]], dtype=np.float32)
    tok = np.array([[[10, 11, 12, 13]]])
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(1, np.int64), 4)
    # -1, -2, then the two -inf ones by candidate index (NaN is candidate 0).
    assert list(token[0, 1:]) == [11, 13, 10, 12]
    assert np.isneginf(score[0, 3]) and np.isneginf(score[0, 4])


def test_scores_accumulate_in_float32_root_down():
    """-1 - 1e-9 rounds to -1 in float32, so every depth-2 node ties with the
    depth-1 nodes: depth 1 first, then parents in order, then candidates.  (In
    float64 the depth-2 nodes would order by their second log-prob.)"""
    lp = np.array([[[-1.0, -1.0], [-1e-9, -2e-9]]], dtype=np.float32)
    tok = _unique_tokens(1, 2, 2)
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(1, np.int64), 6)
    assert list(parent[0]) == [-1, 0, 0, 1, 1, 2, 2]
    assert [t % 1000 for t in token[0, 1:]] == [0, 1, 0, 1, 0, 1]
    assert (score[0, 1:] == np.float32(-1.0)).all()


def test_float32_tied_siblings_go_by_log_prob_rank():
    """Under a parent scoring -1, log-probs -2e-9 (candidate 0) and -1e-9
    (candidate 1) both give -1 in float32: the tie goes to the higher
    log-prob, candidate 1, before candidate 0."""
    lp = np.array([[[-1.0, -3.0], [-2e-9, -1e-9]]], dtype=np.float32)
    tok = _unique_tokens(1, 2, 2)
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(1, np.int64), 3)
    # node 1 = depth-1 candidate 0 (-1); then its children (-1, -1) before the
    # other depth-1 candidate (-3).
    assert list(parent[0]) == [-1, 0, 1, 1]
    assert [t % 1000 for t in token[0, 1:]] == [0, 1, 0]
    assert (score[0, 1:] == np.float32(-1.0)).all()


def test_frontier_exhaustion_and_zero_budget():
    lp = np.full((1, 2, 2), -0.5, dtype=np.float32)
    tok = _unique_tokens(1, 2, 2)
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(1, np.int64), 10)
    assert n[0] == 6 and (parent[0, 7:] == -1).all() and (depth[0, 7:] == -1).all()
    parent, token, depth, score, n = best_first_tree(lp, tok, np.array([3]), 0)
    assert n[0] == 0 and parent.shape == (1, 1) and token[0, 0] == 3


@pytest.mark.parametrize("seed", range(4))
def test_tree_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    B, D, K, budget = 4, 12, 6, 63
    lp = np.log(rng.dirichlet(np.full(K, 0.3), size=(B, D))).astype(np.float32)
    lp = -np.sort(-lp, axis=-1)
    tok = rng.integers(0, 163840, size=(B, D, K))
    parent, token, depth, score, n = best_first_tree(lp, tok, np.zeros(B, np.int64), budget)
    for b in range(B):
        for i in range(1, int(n[b]) + 1):
            p = parent[b, i]
            assert 0 <= p < i and depth[b, i] == depth[b, p] + 1
            assert score[b, i] <= score[b, i - 1] or i == 1  # log-probs <= 0
        assert (parent[b, 1:] >= 0).all()  # 6 + 36 + ... candidates: the budget always fills
