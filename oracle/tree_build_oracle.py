"""CPU oracle for the best-first draft-tree builder (the step before verify).

TEST INFRASTRUCTURE ONLY.  A plain, slow, obviously correct statement of what
the HIP library's tree builder computes.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it; the product path never
does.  It shares no code with the HIP path and imports nothing from it.

Pages cited (by title, then section):
  [RoPE page]   "Precision as Correctness: The Float64 RoPE Decision in a Custom
                CUDA Inference Engine"
  [Verify page] "The Precision Imperative: Validating Numerical Accuracy in a
                Custom CUDA Attention Kernel"
  [Golden page] "The Golden Reference: A Pivotal Moment in Building a Native
                DDTree Inference Engine"

What the pages fix:
  * The engine builds its draft tree on the GPU, best-first, in place of a
    per-request CPU priority-queue (heap) builder.  [Verify page, "The Context:
    What Led to This Moment"; Golden page, "Context: The Quest for a
    Hyper-Optimized Inference Stack"; RoPE page, "The Broader Context: A Full
    Native Engine from Scratch"]
  * Its kernel tests pass bit-exact against the reference.  [RoPE page and
    Golden page, same sections]
  * A small drafter proposes several candidate tokens per position, and the
    target verifies the tree in one pass.  [RoPE page, "The Broader Context"]

Readings where the pages are silent (each pinned by
tests/test_tree_build_oracle.py):
  * The drafter scores every depth at once (a block drafter): at depth
    d = 1..D it proposes K candidates, token cand_tok[d-1, c] with
    log-probability logp[d-1, c], the same whatever the path above.
  * A node is a path of candidates; its score is the sum of the log-probs
    along the path, accumulated in float32 from the root down (the root
    scores 0).  A NaN log-prob counts as -inf.
  * Best-first: the frontier starts as the root's children; `budget` times,
    the best frontier node joins the tree (next node index) and its K
    children join the frontier (none past depth D).
  * Candidates are ranked at their depth: higher log-prob first, equal ones
    by index (the drafter's top-K order; for sorted input the rank is the
    index).
  * "Best" is a total order: higher score; on equal scores the smaller depth,
    then the smaller parent index, then the smaller candidate rank.  (Two
    siblings can tie after float32 rounding although their log-probs differ;
    then the higher log-prob goes first.)
  * Output slot 0 is the root (parent -1, depth 0, score 0, token root_tok).
    If the frontier empties first (K^1 + ... + K^D < budget), the remaining
    slots hold parent -1, token -1, depth -1, score -inf, and n_nodes counts
    the drafted nodes (slots 1 .. n_nodes).
"""
from __future__ import annotations

import heapq

import numpy as np


def best_first_tree(logp, cand_tok, root_tok, budget: int):
    """Build one tree per batch entry.

    logp [B, D, K] float (any float dtype; read as float32), cand_tok [B, D, K]
    int, root_tok [B] int, budget >= 0.

    Returns (parent, token, depth, score) each [B, budget + 1] (int64, int64,
    int64, float32) and n_nodes [B] int64.
    """
    lp = np.asarray(logp, dtype=np.float32)
    tok = np.asarray(cand_tok)
    B, D, K = lp.shape
    lp = np.where(np.isnan(lp), np.float32(-np.inf), lp).astype(np.float32)
    # rank[b, d, c]: position of candidate c in a stable sort by descending log-prob.
    rank = np.empty((B, D, K), dtype=np.int64)
    for b in range(B):
        for d in range(D):
            rank[b, d, np.argsort(-lp[b, d].astype(np.float64), kind="stable")] = np.arange(K)
    q = budget + 1
    parent = np.full((B, q), -1, dtype=np.int64)
    token = np.full((B, q), -1, dtype=np.int64)
    depth = np.full((B, q), -1, dtype=np.int64)
    score = np.full((B, q), -np.inf, dtype=np.float32)
    n_nodes = np.zeros(B, dtype=np.int64)
    for b in range(B):
        token[b, 0] = int(np.asarray(root_tok)[b])
        depth[b, 0] = 0
        score[b, 0] = np.float32(0.0)
        heap = []

        def push_children(node):
            d = int(depth[b, node])
            if d >= D:
                return
            for c in range(K):
                s = np.float32(score[b, node] + lp[b, d, c])  # one float32 add
                # heapq pops the smallest: negate the score; the rest ascend.
                heapq.heappush(heap, (-float(s), d + 1, node, int(rank[b, d, c]), c))

        push_children(0)
        n = 0
        while n < budget and heap:
            neg_s, d, par, _, c = heapq.heappop(heap)
            n += 1
            parent[b, n] = par
            depth[b, n] = d
            token[b, n] = int(tok[b, d - 1, c])
            score[b, n] = np.float32(-neg_s)
            push_children(n)
        n_nodes[b] = n
    return parent, token, depth, score, n_nodes
