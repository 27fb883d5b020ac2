"""tv_verify_attn_noalloc against tv_verify_attn: the same kernels and plan,
with the split-kv partials in the library's static device array instead of a
caller workspace.  Two calls in a row, the second smaller, each checked
against the workspace entry point (bit for bit: no atomics, same launch) and
against the float64 oracle at the usual tolerance."""
import numpy as np
import pytest
import torch

from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W
from tvcompare import errors

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-5, max_rel=1e-2), "bf16": dict(max_rel=2e-2)}


def _inputs(B, H, q, P, dt, seed):
    rng = np.random.default_rng(seed)
    sc = 0.5 if dt == "bf16" else 1.0
    q_lat = (rng.standard_normal((B, q, H, 512), dtype=np.float32) * sc).astype(np.float32)
    q_rope = (rng.standard_normal((B, q, H, 64), dtype=np.float32) * sc).astype(np.float32)
    c_kv = (rng.standard_normal((B, P + q, 512), dtype=np.float32) * sc).astype(np.float32)
    k_rope = (rng.standard_normal((B, P + q, 64), dtype=np.float32) * sc).astype(np.float32)
    if dt == "bf16":
        c_kv, k_rope = W.f32_to_bf16_bits(c_kv), W.f32_to_bf16_bits(k_rope)
    parent = np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)
    return q_lat, q_rope, c_kv, k_rope, parent


def _cache(a, dt):
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _one(B, H, q, P, dt, seed):
    print(f"noalloc B={B} H={H} q={q} P={P} {dt}", flush=True)
    q_lat, q_rope, c_kv, k_rope, parent = _inputs(B, H, q, P, dt, seed)
    code = tv.TV_BF16 if dt == "bf16" else tv.TV_F32
    need = tv.workspace_size(B, H, q, P, 512, 64, code)
    assert 0 < need <= tv.TV_NOALLOC_SCRATCH_BYTES  # the case uses the scratch
    args = (torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(c_kv, dt), _cache(k_rope, dt),
            torch.from_numpy(parent).cuda(), P, 0.04)
    out_n = torch.full((B, q, H, 512), float("nan"), device="cuda")
    lse_n = torch.full((B, q, H), float("nan"), device="cuda")
    tv.verify_attn_noalloc(*args, out=out_n, lse=lse_n)
    out_w, lse_w = tv.verify_attn(*args, return_lse=True)
    torch.cuda.synchronize()
    out_n, lse_n, out_w, lse_w = (t.cpu().numpy() for t in (out_n, lse_n, out_w, lse_w))
    assert np.array_equal(out_n, out_w) and np.array_equal(lse_n, lse_w)
    ref, _ = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, dt),
                           O.as_f64(k_rope, dt), parent, P, 0.04)
    e = errors(out_n, ref)
    assert e["max_rel"] <= TOL[dt]["max_rel"], e
    if "max_abs" in TOL[dt]:
        assert e["max_abs"] <= TOL[dt]["max_abs"], e


def test_noalloc_matches_workspace_entry_two_calls():
    _one(2, 64, 33, 6000, "bf16", seed=1)   # every row block split into kv pieces
    _one(1, 16, 17, 3000, "f32", seed=2)    # smaller, the fp32 matrix-core kernel


def test_noalloc_refuses_oversized_shapes():
    assert tv.workspace_size(4, 64, 33, 200000, 512, 64, tv.TV_BF16) > tv.TV_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((4, 33, 64, 512), device="cuda")
    with pytest.raises(tv.TVError) as ei:
        tv.verify_attn_noalloc(q, torch.zeros((4, 33, 64, 64), device="cuda"),
                               torch.zeros((4, 200033, 512), dtype=torch.bfloat16, device="cuda"),
                               torch.zeros((4, 200033, 64), dtype=torch.bfloat16, device="cuda"),
                               torch.zeros((4, 33), dtype=torch.int32, device="cuda"), 200000, 0.04, out=q)
    assert ei.value.code == tv.TV_ERR_UNSUPPORTED
