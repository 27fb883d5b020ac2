"""CPU oracle for the tree-verify MLA-absorb attention step.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, float64 statement of
what the HIP library computes.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does.
It shares no code with the HIP path and imports nothing from it.

Pages cited (by title, then section):
  [RoPE page]   "Precision as Correctness: The Float64 RoPE Decision in a Custom
                CUDA Inference Engine"
  [Verify page] "The Precision Imperative: Validating Numerical Accuracy in a
                Custom CUDA Attention Kernel"
  [Golden page] "The Golden Reference: A Pivotal Moment in Building a Native
                DDTree Inference Engine"

The method is exact attention restricted to a mask, so the oracle is that
definition written out (no tiling, no online softmax, no fusion):

  1. NeoX RoPE of the rope slices, angle/cos/sin/rotation in float64, one
     rounding to the storage type.  [RoPE page, "The Message", "The Float64
     Decision", "What Input Knowledge Is Required" item 1]
  2. Scores in the absorbed latent space: q_lat . c_kv[j] + q_rope . k_rope[j],
     times sm_scale; one latent row per key, shared by every head.
     [Golden page, "The Absorb Form of MLA"; Verify page, "Input Knowledge
     Required"]
  3. Visibility: the whole prefix, plus the node's ancestors and itself.
     [Verify page, "The Context: What Led to This Moment"; Golden page,
     "Principled Abstraction"]
  4. Softmax over the visible keys, then the probability-weighted sum of the
     latent rows (the output stays in latent space; no w_vc).  [Verify page,
     "The Context: What Led to This Moment" (score, normalise, accumulate)]

Readings where the pages are silent (each pinned by tests/test_oracle.py):
  * Tree = parent array, node 0 the root, parents precede children; node m
    occupies kv row prefix_len + m (kv_len = prefix + q_len, from the printed
    shapes on the Verify page, "The Message in Full").
  * Node positions are prefix_len + depth(node): siblings share a position.
  * inv_freq[k] = 1 / theta**(2k/d_r), NeoX pairing (x[k], x[k + d_r/2]).
  * lse = m + ln(sum exp(s - m)) is returned next to the output.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# Trees, positions and visibility
# ----------------------------------------------------------------------------
def validate_tree(parent) -> np.ndarray:
    """Check parent arrays [B, q_len] (or [q_len]); return them as int64 [B, q_len].

    Valid: parent[0] == -1 and 0 <= parent[i] < i for i >= 1 (node 0 is the root
    and nodes are in topological order).  Raises ValueError otherwise.
    """
    p = np.asarray(parent)
    if p.ndim == 1:
        p = p[None, :]
    if p.ndim != 2 or p.shape[1] < 1:
        raise ValueError(f"parent must be [B, q_len] with q_len >= 1, got shape {p.shape}")
    p = p.astype(np.int64)
    for b in range(p.shape[0]):
        if p[b, 0] != -1:
            raise ValueError(f"batch {b}: node 0 must be the root (parent -1), got {p[b, 0]}")
        for i in range(1, p.shape[1]):
            if not (0 <= p[b, i] < i):
                raise ValueError(f"batch {b}: parent[{i}] = {p[b, i]} is not an earlier node")
    return p


def tree_depths(parent) -> np.ndarray:
    """depth[root] = 0, depth[i] = depth[parent[i]] + 1."""
    p = validate_tree(parent)
    d = np.zeros_like(p)
    for b in range(p.shape[0]):
        for i in range(1, p.shape[1]):
            d[b, i] = d[b, p[b, i]] + 1
    return d


def node_positions(parent, prefix_len: int) -> np.ndarray:
    """Rotary position of each tree node: prefix_len + depth (siblings share one)."""
    return prefix_len + tree_depths(parent)


def key_positions(parent, prefix_len: int) -> np.ndarray:
    """Position of every kv row: j for prefix rows, prefix_len + depth(m) for node m."""
    npos = node_positions(parent, prefix_len)
    B = npos.shape[0]
    pre = np.broadcast_to(np.arange(prefix_len, dtype=np.int64), (B, prefix_len))
    return np.concatenate([pre, npos], axis=1)


def ancestors_of(parent_row, i: int) -> list:
    """Nodes on the path from node i up to the root, i itself included (explicit walk)."""
    out = []
    n = int(i)
    while n != -1:
        out.append(n)
        n = int(parent_row[n])
    return out


def visibility(parent, prefix_len: int) -> np.ndarray:
    """vis[b, i, j]: may tree node i attend to kv row j?

    Every prefix row is visible; of the tree rows (j = prefix_len + m) only the
    node's ancestors and the node itself are.
    """
    p = validate_tree(parent)
    B, q = p.shape
    vis = np.zeros((B, q, prefix_len + q), dtype=bool)
    vis[:, :, :prefix_len] = True
    for b in range(B):
        for i in range(q):
            for m in ancestors_of(p[b], i):
                vis[b, i, prefix_len + m] = True
    return vis


# ----------------------------------------------------------------------------
# Storage types
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to their exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor ("f32" array or "bf16" bit patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_f32(x) -> np.ndarray:
    """One round-to-nearest-even from float64 to fp32 (returned as float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """One round-to-nearest-even from float64 straight to bf16 (8 significant bits).

    Written as mantissa scaling + rint (ties to even), so there is a single
    rounding (no detour through fp32).  Values are assumed inside bf16's normal
    range, as every input here is.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return round_to_f32(x)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def f64_to_bf16_bits(x) -> np.ndarray:
    """Bit patterns of float64 values that are already exact bf16 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# NeoX RoPE  [RoPE page, "The Message"; "The Float64 Decision";
#             "What Input Knowledge Is Required" item 1]
# ----------------------------------------------------------------------------
def rope_inv_freq(d_r: int, theta: float) -> np.ndarray:
    """inv_freq[k] = 1 / theta**(2k / d_r) for k < d_r/2, in float64."""
    if d_r % 2:
        raise ValueError("d_r must be even")
    k = np.arange(d_r // 2, dtype=np.float64)
    return 1.0 / theta ** (2.0 * k / d_r)


def rope_neox(x, pos, theta: float) -> np.ndarray:
    """NeoX rotation of x[..., d_r] at integer positions pos[...], unrounded float64.

    The feature axis is split into halves x1 = x[:d/2], x2 = x[d/2:]; pair k,
    i.e. (x1[k], x2[k]), turns by the angle pos * inv_freq[k]:
        y1 = x1 cos - x2 sin,   y2 = x2 cos + x1 sin.
    Angle, cos, sin and the rotation are all float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = rope_inv_freq(d, theta)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_neox_stored(x, pos, theta: float, dtype: str) -> np.ndarray:
    """rope_neox followed by the single rounding to the storage type (as float64)."""
    return round_to(rope_neox(x, pos, theta), dtype)


# ----------------------------------------------------------------------------
# Tree-verify MLA-absorb attention
# ----------------------------------------------------------------------------
def _check_shapes(q_lat, q_rope, c_kv, k_rope, parent, prefix_len):
    B, q, H, d_c = q_lat.shape
    d_r = q_rope.shape[-1]
    kv = prefix_len + q
    if q_rope.shape != (B, q, H, d_r):
        raise ValueError(f"q_rope shape {q_rope.shape} != {(B, q, H, d_r)}")
    if c_kv.shape != (B, kv, d_c):
        raise ValueError(f"c_kv shape {c_kv.shape} != {(B, kv, d_c)}")
    if k_rope.shape != (B, kv, d_r):
        raise ValueError(f"k_rope shape {k_rope.shape} != {(B, kv, d_r)}")
    if np.asarray(parent).shape != (B, q):
        raise ValueError(f"parent shape {np.asarray(parent).shape} != {(B, q)}")
    if prefix_len < 0:
        raise ValueError("prefix_len must be >= 0")


def verify_attn(q_lat, q_rope, c_kv, k_rope, parent, prefix_len: int, sm_scale: float,
                return_probs: bool = False, batches=None):
    """Tree-verify attention in the absorbed latent space, float64.

    Inputs are float64 arrays holding the stored values (rope slices already
    rotated): q_lat [B,q,H,d_c], q_rope [B,q,H,d_r], c_kv [B,kv,d_c],
    k_rope [B,kv,d_r], parent [B,q].  Returns out [B,q,H,d_c] and lse [B,q,H]
    (and probs [B,q,H,kv] if asked).  ``batches`` restricts the work to a
    subset of batch entries (the other entries of the result are NaN).
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    _check_shapes(q_lat, q_rope, c_kv, k_rope, parent, prefix_len)
    vis = visibility(parent, prefix_len)
    B, q, H, d_c = q_lat.shape
    kv = prefix_len + q
    out = np.full((B, q, H, d_c), np.nan)
    lse = np.full((B, q, H), np.nan)
    probs = np.full((B, q, H, kv), np.nan) if return_probs else None
    for b in (range(B) if batches is None else batches):
        # Scores: latent part plus rope part, one shared latent row per key.
        s = np.matmul(q_lat[b], c_kv[b].T) + np.matmul(q_rope[b], k_rope[b].T)  # [q,H,kv]
        s = sm_scale * s
        s = np.where(vis[b][:, None, :], s, NEG_INF)
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=-1, keepdims=True)
        p = e / l
        out[b] = np.matmul(p, c_kv[b])
        lse[b] = (m + np.log(l))[..., 0]
        if return_probs:
            probs[b] = p
    if return_probs:
        return out, lse, probs
    return out, lse


def verify_step(q_lat, q_rope_raw, c_kv, k_rope_raw, parent, prefix_len: int, theta: float,
                sm_scale: float, kv_dtype: str = "f32", batches=None) -> dict:
    """The whole step: RoPE at tree positions, then tree-verify attention.

    Inputs are the stored values (fp32 arrays; for kv_dtype "bf16" the cache
    arrays are uint16 bf16 bit patterns), rope slices unrotated.  Query rope
    rows turn at prefix_len + depth(node); key rows turn at their own index for
    the prefix and at prefix_len + depth(m) for tree node m.  Each rotated
    slice is rounded once to its storage type (fp32 for queries, kv_dtype for
    keys) before it is used.
    """
    q_lat = as_f64(q_lat, "f32")
    q_rope = as_f64(q_rope_raw, "f32")
    c_kv = as_f64(c_kv, kv_dtype)
    k_rope = as_f64(k_rope_raw, kv_dtype)
    pos_q = node_positions(parent, prefix_len)
    pos_k = key_positions(parent, prefix_len)
    q_rot = rope_neox_stored(q_rope, pos_q[:, :, None], theta, "f32")
    k_rot = rope_neox_stored(k_rope, pos_k, theta, kv_dtype)
    out, lse = verify_attn(q_lat, q_rot, c_kv, k_rot, parent, prefix_len, sm_scale,
                           batches=batches)
    return dict(out=out, lse=lse, q_rope=q_rot, k_rope=k_rot, pos_q=pos_q, pos_k=pos_k)
