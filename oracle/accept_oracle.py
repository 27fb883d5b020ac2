"""CPU oracle for the steps right after verify: greedy tokens, greedy tree
accept, and post-verify KV compaction.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct statements of what
the HIP library computes for these steps.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it; the product path
never does.  It shares no code with the HIP path and imports nothing from it.

Pages cited (by title, then section):
  [RoPE page]   "Precision as Correctness: The Float64 RoPE Decision in a Custom
                CUDA Inference Engine"
  [Golden page] "The Golden Reference: A Pivotal Moment in Building a Native
                DDTree Inference Engine"

What the pages fix:
  * The engine has a greedy tree-accept kernel, and its KV cache is compacted
    after verification.  [RoPE page, "The Broader Context: A Full Native Engine
    from Scratch"; Golden page, "Context: The Quest for a Hyper-Optimized
    Inference Stack"]
  * The invariant: the speculative loop's greedy output equals autoregressive
    greedy output token for token.  [RoPE page, "The Broader Context: ...";
    Golden page, "Context: The Quest for a Hyper-Optimized Inference Stack"]
  * A step involves a root token, draft tokens and a bonus token.  [Golden
    page, "Recursive Refinement of the Decode Loop Design"]

Readings where the pages are silent (each pinned by tests/test_accept_oracle.py):
  * The target's token after node i is the argmax of its logits at node i
    ("greedy"); ties take the lowest index, a NaN counts as the largest value
    (the first NaN wins), and -0.0 equals +0.0.
  * Accept: node 0 (the root) is already committed.  From the current node,
    the next token the target would emit is target[cur]; the walk moves to the
    child of cur whose draft token equals it (the lowest-index child if several
    do) and stops when none does.  The bonus token is target[last accepted
    node].  A step commits the accepted draft tokens and then the bonus token.
  * Compaction: after acceptance the accepted nodes' latent and rope rows move
    to consecutive rows right after the root, row prefix_len + k taking node
    path[k]'s row (k = 1 .. accept_len); every other row is left as it was.
    Node path[k] has depth k, so its rope row (rotated at prefix_len + depth)
    is already rotated for its new row.
"""
from __future__ import annotations

import numpy as np

from oracle.tv_oracle import validate_tree


def greedy_tokens(logits) -> np.ndarray:
    """Argmax over the last axis (the vocabulary) of float logits; int64.

    numpy's argmax is the plain definition: first index of the maximum, a NaN
    counts as the maximum (first NaN wins), -0.0 and +0.0 compare equal.
    bf16 logits are passed as their float values (exact in float64).
    """
    x = np.asarray(logits, dtype=np.float64)
    return np.argmax(x, axis=-1).astype(np.int64)


def tree_accept(parent, draft_tok, target_tok):
    """Greedy acceptance of one draft tree per batch entry.

    parent [B, q] (validated as for verify), draft_tok [B, q] (node 0's entry
    is the root token and is not compared), target_tok [B, q] (the target's
    greedy token after each node).

    Returns (path [B, q] int64 with path[b, 0] = 0, the accepted nodes in
    order, then -1; accept_len [B] = number of accepted draft nodes;
    bonus [B] = target_tok at the last accepted node).
    """
    p = validate_tree(parent)
    d = np.asarray(draft_tok).reshape(p.shape).astype(np.int64)
    t = np.asarray(target_tok).reshape(p.shape).astype(np.int64)
    B, q = p.shape
    path = np.full((B, q), -1, dtype=np.int64)
    accept_len = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    for b in range(B):
        cur, n = 0, 0
        path[b, 0] = 0
        while True:
            want = t[b, cur]
            nxt = -1
            for c in range(1, q):  # lowest-index child carrying the wanted token
                if p[b, c] == cur and d[b, c] == want:
                    nxt = c
                    break
            if nxt < 0:
                break
            n += 1
            path[b, n] = nxt
            cur = nxt
        accept_len[b] = n
        bonus[b] = t[b, cur]
    return path, accept_len, bonus


def committed_tokens(draft_tok, path, accept_len, bonus):
    """Tokens a step commits per batch entry: accepted drafts, then the bonus."""
    d = np.asarray(draft_tok)
    out = []
    for b in range(len(accept_len)):
        toks = [int(d[b, path[b, k]]) for k in range(1, int(accept_len[b]) + 1)]
        out.append(toks + [int(bonus[b])])
    return out


def kv_compact(c_kv, k_rope, path, accept_len, prefix_len: int):
    """Post-verify compaction of [B, kv_rows, d] caches (copies; inputs untouched).

    Row prefix_len + k of entry b takes row prefix_len + path[b, k] for
    k = 1 .. accept_len[b]; all other rows are unchanged.
    """
    c = np.array(c_kv, copy=True)
    r = np.array(k_rope, copy=True)
    src_c = np.asarray(c_kv)
    src_r = np.asarray(k_rope)
    P = int(prefix_len)
    for b in range(len(accept_len)):
        for k in range(1, int(accept_len[b]) + 1):
            m = int(path[b, k])
            c[b, P + k] = src_c[b, P + m]
            r[b, P + k] = src_r[b, P + m]
    return c, r
