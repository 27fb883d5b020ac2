"""Error measures used by the parity tests.

max_abs = max |g - r| over every element.
max_rel = max |g - r| / max(|r|, rms(r_row)), where r_row is the d_c-vector of
          the same (batch, node, head) output row.  The row floor keeps a
          single near-zero reference element among ~10^7 from deciding
          pass or fail; the raw element-wise ratio is reported beside it.
"""
from __future__ import annotations

import numpy as np


def errors(got, ref) -> dict:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite values in the result"
    d = np.abs(g - r)
    row_rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    floor = np.maximum(np.abs(r), row_rms)
    with np.errstate(divide="ignore", invalid="ignore"):
        raw = np.where(np.abs(r) > 0, d / np.abs(r), np.where(d > 0, np.inf, 0.0))
        rel = np.where(floor > 0, d / floor, np.where(d > 0, np.inf, 0.0))
    return {"max_abs": float(d.max(initial=0.0)), "max_rel": float(rel.max(initial=0.0)),
            "max_raw_rel": float(raw.max(initial=0.0))}


def pass_line(tag: str, shape: str, e: dict) -> str:
    return (f"PASS {tag} {shape} max_abs={e['max_abs']:.2e} max_rel={e['max_rel']:.2e} "
            f"(raw elementwise {e['max_raw_rel']:.2e})")


def ulp_diff_f32(a, b) -> np.ndarray:
    """|a - b| in units in the last place of fp32 (same-sign finite inputs)."""
    ia = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def ulp_diff_bf16(a_bits, b_bits) -> np.ndarray:
    ia = np.asarray(a_bits, dtype=np.uint16).astype(np.int64)
    ib = np.asarray(b_bits, dtype=np.uint16).astype(np.int64)
    ia = np.where(ia & 0x8000, -(ia & 0x7FFF), ia)
    ib = np.where(ib & 0x8000, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def rope_mismatch(got, ref, x_raw, dtype: str, max_pos: int):
    """Compare a stored RoPE result with the oracle's.

    Both sides round the same float64 rotation once; they may differ only where
    the device's float64 pow/sin/cos differ from the host's in the last bit and
    the rotated value sits near a rounding boundary, or where the rotation
    cancels (x1 cos ~ x2 sin) so a float64-level difference is many storage
    ulps of a tiny result.  A last-bit difference in inv_freq moves the angle
    by up to pos * 2^-52 rad (relative to inv_freq <= 1), and sin/cos/the
    rotation add a few 2^-53, so the allowance is
        |got - ref| <= 1 storage ulp of ref + (|x1| + |x2|) (max_pos + 4) 2^-50.
    Returns (n_beyond_allowance, fraction_not_identical).
    """
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    x = np.abs(np.asarray(x_raw, dtype=np.float64))
    half = x.shape[-1] // 2
    pair = x[..., :half] + x[..., half:]
    pair = np.concatenate([pair, pair], axis=-1)
    if dtype == "bf16":
        e = np.frexp(np.maximum(np.abs(r), 1e-30))[1]
        ulp = np.ldexp(1.0, e - 8)
    else:
        ulp = np.spacing(np.abs(r).astype(np.float32)).astype(np.float64)
    d = np.abs(g - r)
    beyond = int(np.count_nonzero(d > ulp + pair * (max_pos + 4) * 2.0 ** -50))
    return beyond, float(np.count_nonzero(d) / d.size)


def lse_bound(kind, ref_lse):
    """Allowed |lse - ref| per row.  f32: scores rounded at ~1e-7 relative,
    and the lse is itself an fp32 number (taken in base 2, then scaled by
    ln 2): 2e-5 plus 2^-20 of |lse| (eight fp32 ulps of a value that size; at
    |lse| ~ 100 a few ulps of the max score alone exceed 2e-5).
    bf16 (the default bf16-cache kernel): scores to fp32 precision, softmax
    weights rounded to fp16 (each within 2^-11 relative, so the log of their
    sum moves by at most ~2^-11): 2^-10 plus 2^-14 of |lse|.  bf16_queries (the
    one-term option): weights rounded to bf16 (2^-8) and each score moved by a
    few 2^-9 of its terms: 2^-8 plus 2^-12 of |lse|."""
    r = np.abs(np.asarray(ref_lse, np.float64))
    if kind == "f32":
        return 2e-5 + 2.0 ** -20 * r
    if kind == "bf16":
        return 2.0 ** -10 + 2.0 ** -14 * r
    if kind == "bf16_queries":
        return 2.0 ** -8 + 2.0 ** -12 * r
    raise ValueError(kind)

