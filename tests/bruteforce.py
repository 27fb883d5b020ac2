"""Scalar brute-force references used to pin the oracle (tests only).

Written independently of oracle/: the ancestor relation comes from a
Warshall transitive closure of the parent relation (not a parent walk), and
every sum is a ``math.fsum`` over Python floats.
"""
from __future__ import annotations

import itertools
import math


def all_recursive_trees(q_len: int):
    """Every parent array with parent[0] = -1 and parent[i] in [0, i-1]: (q_len-1)! trees."""
    for rest in itertools.product(*[range(i) for i in range(1, q_len)]):
        yield [-1, *rest]


def ancestor_closure(parent_row):
    """A[i][j] is True iff node j is node i or one of its ancestors."""
    q = len(parent_row)
    A = [[i == j for j in range(q)] for i in range(q)]
    for i in range(q):
        if parent_row[i] >= 0:
            A[i][parent_row[i]] = True
    for k in range(q):
        for i in range(q):
            if A[i][k]:
                for j in range(q):
                    if A[k][j]:
                        A[i][j] = True
    return A


def visible_scalar(parent_row, prefix_len, i, j):
    if j < prefix_len:
        return True
    return ancestor_closure(parent_row)[i][j - prefix_len]


def verify_attn_scalar(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, sm_scale):
    """Per-element loops; inputs are nested lists / arrays of floats."""
    B = len(q_lat)
    q = len(q_lat[0])
    H = len(q_lat[0][0])
    d_c = len(q_lat[0][0][0])
    d_r = len(q_rope[0][0][0])
    kv = prefix_len + q
    out = [[[[0.0] * d_c for _ in range(H)] for _ in range(q)] for _ in range(B)]
    lse = [[[0.0] * H for _ in range(q)] for _ in range(B)]
    for b in range(B):
        A = ancestor_closure(list(parent[b]))
        for i in range(q):
            keys = [j for j in range(kv) if j < prefix_len or A[i][j - prefix_len]]
            for h in range(H):
                s = []
                for j in keys:
                    dot = math.fsum([float(q_lat[b][i][h][d]) * float(c_kv[b][j][d]) for d in range(d_c)]
                                    + [float(q_rope[b][i][h][d]) * float(k_rope[b][j][d]) for d in range(d_r)])
                    s.append(sm_scale * dot)
                m = max(s)
                e = [math.exp(x - m) for x in s]
                l = math.fsum(e)
                for d in range(d_c):
                    out[b][i][h][d] = math.fsum([e[t] * float(c_kv[b][j][d]) for t, j in enumerate(keys)]) / l
                lse[b][i][h] = m + math.log(l)
    return out, lse


# ----------------------------------------------------------------------------
# Greedy accept, argmax and compaction (independent of oracle/accept_oracle.py)
# ----------------------------------------------------------------------------
def argmax_scalar(row):
    """First index of the largest value; a NaN beats everything (first NaN wins);
    -0.0 and +0.0 are equal.  A plain Python scan."""
    best_i, best = 0, None
    for i, v in enumerate(row):
        v = float(v)
        if best is None:
            best_i, best = i, v
            continue
        if math.isnan(best):
            continue
        if math.isnan(v) or v > best:
            best_i, best = i, v
    return best_i


def accept_scalar(parent_row, draft_row, target_row):
    """Deepest node whose root path follows the target's greedy tokens, found by
    checking every node's whole path (for trees without two siblings carrying
    the same draft token, where that node is unique).

    Returns (path as a list of node indices from the root, bonus token)."""
    q = len(parent_row)
    best = [0]
    for v in range(q):
        chain = [v]
        while chain[-1] != 0:
            chain.append(parent_row[chain[-1]])
        chain.reverse()                      # root ... v
        ok = all(draft_row[chain[k]] == target_row[chain[k - 1]] for k in range(1, len(chain)))
        if ok and len(chain) > len(best):
            best = chain
    return best, target_row[best[-1]]


def compact_scalar(rows, path, accept_len, prefix_len):
    """rows: list of per-row values of one cache entry; returns the compacted list."""
    out = list(rows)
    for k in range(1, accept_len + 1):
        out[prefix_len + k] = rows[prefix_len + path[k]]
    return out
