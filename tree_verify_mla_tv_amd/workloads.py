"""Seeded synthetic inputs for the tree-verify MLA-absorb attention step.

This module only draws random numbers and shapes them: it holds none of the
method's arithmetic (no RoPE, no masking, no softmax).  Both the HIP path and
the CPU oracle are fed from here, so the two never share anything else.

Workloads mirror the test shapes printed on "The Precision Imperative:
Validating Numerical Accuracy in a Custom CUDA Attention Kernel" (section "The
Message in Full": B, H, q_len, kv_len of each verify-attn bundle), with
kv_len = prefix + q_len and q_len = budget + 1, plus one serving-scale shape.

Recipe (fixed, per workload):
  * ``numpy.random.default_rng(seed)``; draw order q_lat, q_rope, c_kv,
    k_rope, then one tree per batch entry.
  * Values are standard normal fp32, times ``scale`` (1.0, or 0.5 for the
    serving-scale workload).
  * A bf16 cache is the fp32 draw rounded to nearest-even bf16; it is carried
    as uint16 bit patterns.
  * q_rope and k_rope are drawn *unrotated*; the step rotates them.
  * Trees are parent arrays: node 0 is the root (parent -1) and every other
    node's parent precedes it (topological order).  Shapes: ``rrt`` (parent
    uniform over all earlier nodes), ``chain`` (parent = i-1), ``wide``
    (parent uniform over the first min(i, 8) nodes), ``branch4`` (parent
    uniform over earlier nodes that still have fewer than 4 children).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

THETA = 10000.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    prefix_len: int
    q_len: int
    d_c: int
    d_r: int
    kv_dtype: str  # "f32" or "bf16"
    tree: str
    seed: int
    scale: float = 1.0
    theta: float = THETA

    @property
    def kv_len(self) -> int:
        return self.prefix_len + self.q_len

    @property
    def sm_scale(self) -> float:
        # 1/sqrt(d_c + d_r), rounded to the fp32 value both sides receive.
        return float(np.float32(1.0 / math.sqrt(self.d_c + self.d_r)))

    def describe(self) -> str:
        return (f"B={self.B} H={self.H} prefix={self.prefix_len} q_len={self.q_len} "
                f"kv_len={self.kv_len} d_c={self.d_c} d_r={self.d_r} kv={self.kv_dtype} "
                f"tree={self.tree}")


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_b3_h8_p1_q5", 3, 8, 1, 5, 64, 32, "f32", "rrt", seed=1),
        Workload("b2_h8_p0_q9", 2, 8, 0, 9, 64, 32, "f32", "rrt", seed=2),
        Workload("b2_h8_p0_q9_chain", 2, 8, 0, 9, 64, 32, "f32", "chain", seed=2),
        Workload("b2_h64_p512_q9", 2, 64, 512, 9, 512, 64, "f32", "rrt", seed=3),
        Workload("b2_h16_p2048_q17", 2, 16, 2048, 17, 512, 64, "f32", "rrt", seed=4),
        Workload("b1_h64_p128_q33_wide", 1, 64, 128, 33, 512, 64, "f32", "wide", seed=4),
        Workload("serve_b32_h64_p8192_q33_bf16", 32, 64, 8192, 33, 512, 64, "bf16",
                 "branch4", seed=5, scale=0.5),
    ]
}

# The serving-scale shape is the throughput workload; the others are parity cases.
SERVING = "serve_b32_h64_p8192_q33_bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to nearest-even bf16; return the uint16 bit patterns.

    Inputs are finite (standard-normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def tree_rrt(q_len: int, rng: np.random.Generator) -> np.ndarray:
    p = np.empty(q_len, np.int32)
    p[0] = -1
    for i in range(1, q_len):
        p[i] = rng.integers(0, i)
    return p


def tree_chain(q_len: int, rng: np.random.Generator | None = None) -> np.ndarray:
    return np.arange(-1, q_len - 1, dtype=np.int32)


def tree_wide(q_len: int, rng: np.random.Generator) -> np.ndarray:
    p = np.empty(q_len, np.int32)
    p[0] = -1
    for i in range(1, q_len):
        p[i] = rng.integers(0, min(i, 8))
    return p


def tree_branch(q_len: int, rng: np.random.Generator, max_children: int = 4) -> np.ndarray:
    p = np.empty(q_len, np.int32)
    p[0] = -1
    children = np.zeros(q_len, np.int64)
    for i in range(1, q_len):
        cand = np.nonzero(children[:i] < max_children)[0]
        par = int(cand[rng.integers(0, len(cand))])
        p[i] = par
        children[par] += 1
    return p


TREES = {"rrt": tree_rrt, "chain": tree_chain, "wide": tree_wide, "branch4": tree_branch}


def make_inputs(w: Workload | str, seed: int | None = None, batch: int | None = None) -> dict:
    """Draw one batch of inputs for workload ``w``.

    Returns numpy arrays: q_lat [B,q,H,d_c] f32, q_rope [B,q,H,d_r] f32,
    c_kv [B,kv,d_c] and k_rope [B,kv,d_r] (f32, or uint16 bf16 bits),
    parent [B,q] int32; plus the scalars prefix_len, theta, sm_scale.
    ``batch`` overrides B (the draw recipe is otherwise unchanged).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if batch is not None:
        w = dataclasses.replace(w, B=batch)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, q, H, kv = w.B, w.q_len, w.H, w.kv_len

    def normal(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if w.scale != 1.0:
            x *= np.float32(w.scale)
        return x

    q_lat = normal((B, q, H, w.d_c))
    q_rope = normal((B, q, H, w.d_r))
    c_kv = normal((B, kv, w.d_c))
    k_rope = normal((B, kv, w.d_r))
    if w.kv_dtype == "bf16":
        c_kv = f32_to_bf16_bits(c_kv)
        k_rope = f32_to_bf16_bits(k_rope)
    tree_fn = TREES[w.tree]
    parent = np.stack([tree_fn(q, rng) for _ in range(B)]).astype(np.int32)
    return dict(q_lat=q_lat, q_rope=q_rope, c_kv=c_kv, k_rope=k_rope, parent=parent,
                prefix_len=w.prefix_len, theta=w.theta, sm_scale=w.sm_scale,
                kv_dtype=w.kv_dtype, workload=w)


# ----------------------------------------------------------------------------
# Inputs of the steps after verify (greedy tokens, tree accept, compaction)
# ----------------------------------------------------------------------------
SERVE_VOCAB = 163840  # a K2-class vocabulary; the pages print only the tiny model's (512)


def make_accept_inputs(parent: np.ndarray, vocab: int, seed: int, logits_dtype: str = "f32",
                       max_accept: int | None = None) -> dict:
    """Synthetic draft tokens and target logits for trees ``parent`` [B, q].

    Recipe: ``numpy.random.default_rng(seed)``.  Each node's draft token is drawn
    uniformly, redrawn until it differs from its earlier siblings' (as a
    best-first drafter's top-k children do).  Logits are N(0,1) fp32 per node
    over the vocabulary.  For each tree a target path is planted: from the root,
    a uniformly chosen child is followed for a depth drawn uniformly from
    [0, min(max depth, max_accept)]; along it, each node's logits get +8 at the
    next path node's draft token (so the target's greedy token there is that
    draft token), and the last path node gets +8 at a token no child of it
    carries.  bf16 logits are the fp32 draw rounded to nearest-even bf16 (uint16
    bit patterns).  Returns draft [B, q] int32, logits [B, q, vocab] (float32 or
    uint16) and the planted depth [B].
    """
    rng = np.random.default_rng(seed)
    p = np.asarray(parent)
    B, q = p.shape
    draft = np.zeros((B, q), dtype=np.int32)
    for b in range(B):
        kids = {}
        for i in range(q):
            taken = kids.setdefault(int(p[b, i]), set())
            while True:
                t = int(rng.integers(0, vocab))
                if t not in taken or i == 0:
                    break
            taken.add(t)
            draft[b, i] = t
    logits = rng.standard_normal((B, q, vocab), dtype=np.float32)
    depth = np.zeros(B, dtype=np.int64)
    for b in range(B):
        children = [[c for c in range(1, q) if p[b, c] == v] for v in range(q)]
        longest = [0] * q
        for v in range(q - 1, -1, -1):
            longest[v] = 1 + max((longest[c] for c in children[v]), default=-1) if children[v] else 0
        cap = longest[0] if max_accept is None else min(longest[0], max_accept)
        want = int(rng.integers(0, cap + 1))
        cur = 0
        for _ in range(want):
            opts = [c for c in children[cur] if longest[c] >= want - depth[b] - 1]
            nxt = opts[int(rng.integers(0, len(opts)))]
            logits[b, cur, draft[b, nxt]] += 8.0
            cur = nxt
            depth[b] += 1
        kid_toks = {int(draft[b, c]) for c in children[cur]}
        while True:
            t = int(rng.integers(0, vocab))
            if t not in kid_toks:
                break
        logits[b, cur, t] += 8.0
    if logits_dtype == "bf16":
        logits = f32_to_bf16_bits(logits)
    return {"draft": draft, "logits": logits, "depth": depth}


# Best-first tree builder at the serving shape: 32 requests, a 32-node draft
# budget (q_len 33), a block drafter proposing its top 8 tokens at each of 16
# depths.
BUILD_DEPTH = 16
BUILD_TOPK = 8


def make_build_inputs(B: int, depth: int, topk: int, seed: int, vocab: int = SERVE_VOCAB,
                      sort: bool = True, alpha: float = 0.3) -> dict:
    """Synthetic drafter proposals for the best-first tree builder.

    Recipe: ``numpy.random.default_rng(seed)``.  At each (request, depth) a
    probability vector over topk + 1 outcomes is drawn from Dirichlet(alpha)
    (the extra outcome stands for the rest of the vocabulary); the log of the
    first topk entries in float32 are the candidates' log-probs, sorted
    descending when ``sort`` (a top-k list), else left in draw order.  Tokens
    are topk distinct ids drawn uniformly from [0, vocab).  Root tokens are
    uniform.  Returns logp [B, depth, topk] float32, cand_tok [B, depth, topk]
    int32, root_tok [B] int32.
    """
    rng = np.random.default_rng(seed)
    pr = rng.dirichlet(np.full(topk + 1, alpha), size=(B, depth))[..., :topk]
    with np.errstate(divide="ignore"):
        logp = np.log(pr).astype(np.float32)
    if sort:
        logp = -np.sort(-logp, axis=-1)
    tok = np.empty((B, depth, topk), dtype=np.int32)
    for b in range(B):
        for d in range(depth):
            tok[b, d] = rng.choice(vocab, size=topk, replace=False)
    root = rng.integers(0, vocab, size=B).astype(np.int32)
    return {"logp": logp, "cand_tok": tok, "root_tok": root}
