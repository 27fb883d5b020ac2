"""Error measures used by the parity tests.

max_abs = max |g - r| over every element.
max_rel = max |g - r| / max(|r|, rms(r_row)), where r_row is the d_c-vector of
          the same (batch, node, head) output row.  The row floor keeps a
          single near-zero reference element among ~10^7 from deciding the
          verdict; the raw element-wise ratio is reported beside it.
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
