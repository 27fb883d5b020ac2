"""Long-prefix, small-batch verify attention (split kv + merge) against the
float64 oracle, up to a 200k-token prefix, and the drift of the float32
accumulation with prefix length.

The GPU runs every head; the oracle recomputes a few heads (heads are
independent: the same latent rows, their own queries), so the reference stays
within host memory at 200k keys.  Each case prints its errors; the table in the
design notes comes from these lines."""
import numpy as np
import pytest
import torch

from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W
from tvcompare import errors

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-5, max_rel=1e-2), "bf16": dict(max_rel=2e-2)}


def _inputs(B, H, q, P, d_c, d_r, dt, seed):
    rng = np.random.default_rng(seed)
    kv = P + q
    scale = 0.5 if dt == "bf16" else 1.0
    q_lat = (rng.standard_normal((B, q, H, d_c), dtype=np.float32) * scale).astype(np.float32)
    q_rope = (rng.standard_normal((B, q, H, d_r), dtype=np.float32) * scale).astype(np.float32)
    c_kv = (rng.standard_normal((B, kv, d_c), dtype=np.float32) * scale).astype(np.float32)
    k_rope = (rng.standard_normal((B, kv, d_r), dtype=np.float32) * scale).astype(np.float32)
    if dt == "bf16":
        c_kv, k_rope = W.f32_to_bf16_bits(c_kv), W.f32_to_bf16_bits(k_rope)
    parent = np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)
    return q_lat, q_rope, c_kv, k_rope, parent


def _cache(a, dt):
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


CASES = [
    # B, H, q, P, dtype, heads checked[, tv_verify_attn_ex flags]
    (1, 64, 33, 8192, "bf16", (0, 21, 63)),
    (1, 64, 33, 32768, "bf16", (0, 21, 63)),
    (1, 64, 33, 131072, "bf16", (0, 63)),
    (1, 64, 33, 200000, "bf16", (0, 63)),
    (2, 64, 33, 65536, "bf16", (5, 40)),
    (4, 16, 17, 50000, "bf16", (0, 15)),
    (1, 8, 33, 8192, "f32", (0, 7)),
    (1, 8, 33, 32768, "f32", (0, 7)),
    (1, 8, 33, 131072, "f32", (0, 7)),
    (1, 8, 33, 200000, "f32", (0, 7)),
    (1, 8, 33, 200000, "f32", (0, 7), tv.TV_ATTN_F32_WIDE),  # the fp32 kernel's 64-row form
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}{c[4]}" + ("wide" if len(c) > 6 else "")
                                             for c in CASES])
def test_long_prefix(case):
    B, H, q, P, dt, heads = case[:6]
    flags = case[6] if len(case) > 6 else 0
    d_c, d_r = 512, 64
    print(f"long prefix case {case}", flush=True)
    q_lat, q_rope, c_kv, k_rope, parent = _inputs(B, H, q, P, d_c, d_r, dt, seed=P + H + B)
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    out, lse = tv.verify_attn_ex(torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(c_kv, dt),
                                 _cache(k_rope, dt), torch.from_numpy(parent).cuda(), P, sm, flags, return_lse=True)
    torch.cuda.synchronize()
    hs = list(heads)
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat[:, :, hs], "f32"), O.as_f64(q_rope[:, :, hs], "f32"),
                                     O.as_f64(c_kv, dt), O.as_f64(k_rope, dt), parent, P, sm)
    got = out.cpu().numpy()[:, :, hs].astype(np.float64)
    e = errors(got, ref_out)
    el = float(np.max(np.abs(lse.cpu().numpy()[:, :, hs] - ref_lse)))
    print(f"DRIFT dtype={dt} flags={flags} P={P} B={B} H={H} q={q} heads={hs} max_abs={e['max_abs']:.3e} "
          f"max_rel={e['max_rel']:.3e} lse_abs={el:.2e}", flush=True)
    assert e["max_rel"] <= TOL[dt]["max_rel"], e
    if "max_abs" in TOL[dt]:
        assert e["max_abs"] <= TOL[dt]["max_abs"], e
