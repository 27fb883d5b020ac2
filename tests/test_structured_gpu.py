"""Verify attention on structured inputs rather than i.i.d. normals: a few
outlier channels (as in real activations), heavy-tailed latent rows, attention
that is nearly one-hot, and attention that is nearly uniform.  GPU against the
float64 oracle at the usual tolerances."""
import numpy as np
import pytest
import torch

from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W
from tvcompare import errors

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-5, max_rel=1e-2), "bf16": dict(max_rel=2e-2)}


def _cache(a, dt):
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(q_lat, q_rope, c_kv, k_rope, parent, P, sm, dt, tag, flags=0):
    print(tag, flush=True)
    if dt == "bf16":
        c_st, k_st = W.f32_to_bf16_bits(c_kv), W.f32_to_bf16_bits(k_rope)
    else:
        c_st, k_st = c_kv, k_rope
    out, lse = tv.verify_attn_ex(torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(c_st, dt),
                                 _cache(k_st, dt), torch.from_numpy(parent).cuda(), P, sm, flags, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_st, dt),
                                 O.as_f64(k_st, dt), parent, P, sm)
    e = errors(out.cpu().numpy(), ref)
    print(tag, e, flush=True)
    assert e["max_rel"] <= TOL[dt]["max_rel"], (tag, e)
    if "max_abs" in TOL[dt]:
        # absolute bound relative to the output scale (outlier channels are large)
        assert e["max_abs"] <= TOL[dt]["max_abs"] * max(1.0, float(np.abs(ref).max())), (tag, e)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= (1e-4 if dt == "f32" else 2.0 ** -6) * max(
        1.0, float(np.abs(ref_lse).max())), tag


def _base(B, H, q, P, d_c, d_r, seed):
    rng = np.random.default_rng(seed)
    kv = P + q
    q_lat = rng.standard_normal((B, q, H, d_c)).astype(np.float32)
    q_rope = rng.standard_normal((B, q, H, d_r)).astype(np.float32)
    c_kv = rng.standard_normal((B, kv, d_c)).astype(np.float32)
    k_rope = rng.standard_normal((B, kv, d_r)).astype(np.float32)
    parent = np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)
    return rng, q_lat, q_rope, c_kv, k_rope, parent


def _outlier_inputs():
    """Eight latent channels 40x larger than the rest in queries and keys, and
    Student-t (3 degrees of freedom) latent rows."""
    B, H, q, P, d_c, d_r = 2, 16, 33, 2000, 512, 64
    rng, q_lat, q_rope, c_kv, k_rope, parent = _base(B, H, q, P, d_c, d_r, 1)
    ch = rng.choice(d_c, 8, replace=False)
    c_kv = rng.standard_t(3, size=c_kv.shape).astype(np.float32)
    q_lat[..., ch] *= 40.0
    c_kv[..., ch] *= 40.0
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r))) / 40.0
    return q_lat, q_rope, c_kv, k_rope, parent, P, sm


def test_outlier_channels_heavy_tails_f32():
    _run(*_outlier_inputs(), "f32", "outliers f32")


def test_outlier_channels_heavy_tails_f32_wide():
    """The same on the fp32 kernel's 64-row form (TV_ATTN_F32_WIDE)."""
    _run(*_outlier_inputs(), "f32", "outliers f32 64-row", flags=tv.TV_ATTN_F32_WIDE)


def test_outlier_channels_heavy_tails_bf16():
    """The bf16-cache kernel carries each scaled query as two bf16 terms, so
    the dominant score terms keep fp32 precision: within the bf16 bound of
    the oracle (a float64 model of its arithmetic puts it near 1e-2)."""
    _run(*_outlier_inputs(), "bf16", "outliers bf16")


@pytest.mark.xfail(strict=True, reason="TV_ATTN_BF16_QUERIES rounds the scaled queries to one bf16 term: "
                                      "max_rel 0.34 against the oracle on these inputs")
def test_outlier_channels_heavy_tails_bf16_queries():
    """The same inputs through tv_verify_attn_ex with TV_ATTN_BF16_QUERIES
    (one bf16 term per query): each score moves by up to 2^-9 of its terms,
    and with a few dominant channels that alone exceeds the bf16 bound."""
    _run(*_outlier_inputs(), "bf16", "outliers bf16 queries", flags=tv.TV_ATTN_BF16_QUERIES)


# cache dtype and tv_verify_attn_ex flags of each variant
VARIANTS = {"bf16": ("bf16", 0), "f32": ("f32", 0), "f32_wide": ("f32", tv.TV_ATTN_F32_WIDE),
            "bf16_queries": ("bf16", tv.TV_ATTN_BF16_QUERIES)}


@pytest.mark.parametrize("dt", list(VARIANTS))
def test_nearly_one_hot(dt):
    """Each query row equals one visible key row scaled up: its softmax puts
    almost all the weight on that key (scores up to ~60 apart in log2)."""
    B, H, q, P, d_c, d_r = 2, 8, 17, 700, 512, 64
    rng, q_lat, q_rope, c_kv, k_rope, parent = _base(B, H, q, P, d_c, d_r, 2)
    for b in range(B):
        for i in range(q):
            for h in range(H):
                j = int(rng.integers(0, P))
                q_lat[b, i, h] = c_kv[b, j] * 0.5
                q_rope[b, i, h] = k_rope[b, j] * 0.5
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    _run(q_lat, q_rope, c_kv, k_rope, parent, P, sm, VARIANTS[dt][0], f"one-hot {dt}", flags=VARIANTS[dt][1])


@pytest.mark.parametrize("dt", list(VARIANTS))
def test_nearly_uniform(dt):
    """A tiny softmax scale: every visible key weighs about the same, so the
    output is close to the mean of the visible latent rows (long sums of
    nearly equal weights)."""
    B, H, q, P, d_c, d_r = 2, 8, 33, 5000, 512, 64
    rng, q_lat, q_rope, c_kv, k_rope, parent = _base(B, H, q, P, d_c, d_r, 3)
    _run(q_lat, q_rope, c_kv, k_rope, parent, P, 1e-4, VARIANTS[dt][0], f"uniform {dt}", flags=VARIANTS[dt][1])
