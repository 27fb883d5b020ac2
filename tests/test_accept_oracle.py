"""Pins for the accept / argmax / compaction oracle (no GPU).

The main pin is the pages' invariant: a verify step's committed tokens must be
what greedy autoregressive decoding would produce.  A synthetic deterministic
"target model" (the next token is a hash of the token history) stands in for
the model; trees are grown around its greedy continuation with distractor
branches, the target's token at each node is that function of the node's root
path, and the committed tokens must equal the greedy rollout.  Independent
scalar brute forces (tests/bruteforce.py) check the accepted path, argmax's
tie / NaN / signed-zero rules and the compaction.
"""
import hashlib

import numpy as np
import pytest

import bruteforce
from oracle import accept_oracle as A


def _next_token(history, vocab):
    """A deterministic stand-in for the target model's greedy next token."""
    h = hashlib.sha256(np.asarray(history, dtype=np.int64).tobytes()).digest()
    return int.from_bytes(h[:8], "little") % vocab


def _grow_tree(rng, q_len, vocab, root_tok, greedy_depth):
    """Tree with the greedy chain to depth greedy_depth plus random distractors,
    no two siblings carrying the same token.  Returns (parent, draft)."""
    parent, draft = [-1], [root_tok]
    hist = {0: [root_tok]}
    children = {0: set()}
    cur = 0
    for _ in range(greedy_depth):
        if len(parent) >= q_len:
            break
        t = _next_token(hist[cur], vocab)
        parent.append(cur)
        draft.append(t)
        n = len(parent) - 1
        hist[n] = hist[cur] + [t]
        children[cur].add(t)
        children[n] = set()
        cur = n
    while len(parent) < q_len:
        p = int(rng.integers(0, len(parent)))
        t = int(rng.integers(0, vocab))
        if t in children[p]:
            continue
        parent.append(p)
        draft.append(t)
        n = len(parent) - 1
        hist[n] = hist[p] + [t]
        children[p].add(t)
        children[n] = set()
    # Shuffle into a random topological order (parents still precede children).
    q = len(parent)
    order = [0]
    pending = list(range(1, q))
    while pending:
        ready = [v for v in pending if parent[v] in order]
        v = ready[int(rng.integers(0, len(ready)))]
        order.append(v)
        pending.remove(v)
    new_of = {old: new for new, old in enumerate(order)}
    parent2 = [-1] + [new_of[parent[old]] for old in order[1:]]
    draft2 = [draft[old] for old in order]
    target2 = [_next_token(hist[old], vocab) for old in order]
    return parent2, draft2, target2


@pytest.mark.parametrize("seed", range(12))
def test_committed_tokens_equal_greedy_rollout(seed):
    rng = np.random.default_rng(seed)
    vocab = int(rng.choice([7, 50, 1000]))
    B, q = 4, int(rng.integers(2, 34))
    parents, drafts, targets, roots = [], [], [], []
    for b in range(B):
        root = int(rng.integers(0, vocab))
        p, d, t = _grow_tree(rng, q, vocab, root, int(rng.integers(0, q)))
        parents.append(p); drafts.append(d); targets.append(t); roots.append(root)
    path, n, bonus = A.tree_accept(parents, drafts, targets)
    committed = A.committed_tokens(np.array(drafts), path, n, bonus)
    for b in range(B):
        hist = [roots[b]]
        for _ in range(n[b] + 1):
            hist.append(_next_token(hist, vocab))
        assert committed[b] == hist[1:], (b, committed[b], hist[1:])
        bf_path, bf_bonus = bruteforce.accept_scalar(parents[b], drafts[b], targets[b])
        assert list(path[b, :n[b] + 1]) == bf_path and int(bonus[b]) == bf_bonus
        assert np.all(path[b, n[b] + 1:] == -1)


def test_accept_special_cases():
    # Root only: nothing to accept, the bonus is the target's token after the root.
    path, n, bonus = A.tree_accept([[-1]], [[5]], [[9]])
    assert n.tolist() == [0] and bonus.tolist() == [9] and path.tolist() == [[0]]
    # A chain whose every draft matches: all accepted.
    par = [[-1, 0, 1, 2]]
    path, n, bonus = A.tree_accept(par, [[0, 11, 12, 13]], [[11, 12, 13, 14]])
    assert n.tolist() == [3] and path.tolist() == [[0, 1, 2, 3]] and bonus.tolist() == [14]
    # No child matches the root's token.
    path, n, bonus = A.tree_accept([[-1, 0, 0]], [[0, 3, 4]], [[5, 1, 1]])
    assert n.tolist() == [0] and bonus.tolist() == [5] and path.tolist() == [[0, -1, -1]]
    # Two siblings with the matching token: the lower index is taken, even when
    # the other sibling's subtree would go deeper.
    par = [[-1, 0, 0, 2]]
    drf = [[0, 7, 7, 8]]
    tgt = [[7, 1, 8, 2]]
    path, n, bonus = A.tree_accept(par, drf, tgt)
    assert path.tolist() == [[0, 1, -1, -1]] and n.tolist() == [1] and bonus.tolist() == [1]
    # A match below a non-matching node is not reachable.
    path, n, bonus = A.tree_accept([[-1, 0, 1]], [[0, 3, 4]], [[9, 4, 6]])
    assert n.tolist() == [0] and bonus.tolist() == [9]


@pytest.mark.parametrize("seed", range(6))
def test_argmax_matches_scalar_scan(seed):
    rng = np.random.default_rng(100 + seed)
    rows = rng.integers(-3, 4, size=(20, 37)).astype(np.float64)  # many ties
    rows[3, 5] = np.nan
    rows[3, 9] = np.nan
    rows[4] = -np.inf
    rows[5, :] = 0.0
    rows[5, 7] = -0.0
    rows[6, 2] = np.inf
    rows[7, 0] = -0.0
    rows[7, 1:] = -1.0
    rows[7, 30] = 0.0
    got = A.greedy_tokens(rows)
    want = [bruteforce.argmax_scalar(r) for r in rows]
    assert got.tolist() == want
    assert got[3] == 5 and got[4] == 0 and got[5] == 0 and got[6] == 2 and got[7] == 0


@pytest.mark.parametrize("seed", range(6))
def test_compaction_matches_scalar(seed):
    rng = np.random.default_rng(200 + seed)
    B, P, q, dc, dr = 3, int(rng.integers(0, 9)), int(rng.integers(1, 12)), 5, 3
    kv = P + q + int(rng.integers(0, 3))      # rows past the tree stay as they are
    c_kv = rng.standard_normal((B, kv, dc))
    k_rope = rng.standard_normal((B, kv, dr))
    parent = [[-1] + [int(rng.integers(0, i)) for i in range(1, q)] for _ in range(B)]
    draft = rng.integers(0, 4, size=(B, q))
    target = rng.integers(0, 4, size=(B, q))
    path, n, _ = A.tree_accept(parent, draft, target)
    c2, r2 = A.kv_compact(c_kv, k_rope, path, n, P)
    for b in range(B):
        want_c = bruteforce.compact_scalar(list(c_kv[b]), list(path[b]), int(n[b]), P)
        want_r = bruteforce.compact_scalar(list(k_rope[b]), list(path[b]), int(n[b]), P)
        assert np.array_equal(c2[b], np.array(want_c)) and np.array_equal(r2[b], np.array(want_r))
        # Untouched: the prefix, the root, and every row past the accepted ones.
        assert np.array_equal(c2[b, :P + 1], c_kv[b, :P + 1])
        assert np.array_equal(c2[b, P + 1 + n[b]:], c_kv[b, P + 1 + n[b]:])


def test_compaction_identity_cases():
    c = np.arange(2 * 6 * 2, dtype=np.float64).reshape(2, 6, 2)
    r = -c[..., :1]
    full = np.array([[0, 1, 2, 3], [0, 1, 2, 3]])
    c2, r2 = A.kv_compact(c, r, full, np.array([3, 0]), 2)
    assert np.array_equal(c2, c) and np.array_equal(r2, r)
    # Hand example: prefix 1, accepted nodes 2 then 3 move to rows 2 and 3.
    c = np.arange(6, dtype=np.float64).reshape(1, 6, 1)
    c2, _ = A.kv_compact(c, c, np.array([[0, 2, 3, -1]]), np.array([2]), 1)
    assert c2[0, :, 0].tolist() == [0.0, 1.0, 3.0, 4.0, 4.0, 5.0]


def test_accept_mutations_are_caught(monkeypatch):
    """Plausible slips in the walk are caught by the invariant pin."""
    rng = np.random.default_rng(7)
    cases = [_grow_tree(rng, 20, 50, 3, 8) for _ in range(6)]
    par = [c[0] for c in cases]; drf = [c[1] for c in cases]; tgt = [c[2] for c in cases]
    good = A.tree_accept(par, drf, tgt)
    # Comparing the child's draft with target[child] instead of target[cur].
    def wrong(parent, draft_tok, target_tok):
        p = np.asarray(parent); d = np.asarray(draft_tok); t = np.asarray(target_tok)
        B, q = p.shape
        path = np.full((B, q), -1); n = np.zeros(B, int); bonus = np.zeros(B, int)
        for b in range(B):
            cur, k = 0, 0
            path[b, 0] = 0
            while True:
                nxt = next((c for c in range(1, q) if p[b, c] == cur and d[b, c] == t[b, c]), -1)
                if nxt < 0:
                    break
                k += 1; path[b, k] = nxt; cur = nxt
            n[b] = k; bonus[b] = t[b, cur]
        return path, n, bonus
    bad = wrong(par, drf, tgt)
    assert not (np.array_equal(bad[0], good[0]) and np.array_equal(bad[2], good[2]))
    for b in range(len(cases)):
        bf_path, _ = bruteforce.accept_scalar(par[b], drf[b], tgt[b])
        assert list(good[0][b, :good[1][b] + 1]) == bf_path
