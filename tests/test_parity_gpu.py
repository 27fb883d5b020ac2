"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Tolerances (per output element; max_rel uses the row floor of tvcompare):
  fp32 cache:  max_abs <= 1e-5 and max_rel <= 1e-2
  bf16 cache:  max_rel <= 2e-2
  lse:         2e-5 + 2^-20 |lse| (fp32 cache); 2^-10 + 2^-14 |lse| (bf16 cache,
               default kernel: the weights are fp16 matrix-core operands);
               2^-8 + 2^-12 |lse| (bf16 cache with TV_ATTN_BF16_QUERIES: bf16
               weights)
RoPE: both sides round the same float64 rotation once, so most values agree
bit for bit; a difference is allowed where the device's float64 pow/sin/cos
differ from the host's in the last bit, bounded by one storage ulp plus the
cancellation allowance of tvcompare.rope_mismatch, and the fraction of
values that differ at all is capped.
"""
import zlib

import numpy as np
import pytest
import torch

from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W
from tvcompare import errors, lse_bound, pass_line, rope_mismatch

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-5, max_rel=1e-2), "bf16": dict(max_rel=2e-2), "bf16_queries": dict(max_rel=2e-2)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tv.load()


def cuda_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def cuda_cache(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return cuda_f32(a)


def cache_numpy(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_out(tag, shape, out, lse, ref_out, ref_lse, dtype, rows=None):
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        out, lse, ref_out, ref_lse = out[rows], lse[rows], ref_out[rows], ref_lse[rows]
    e = errors(out, ref_out)
    tol = TOL[dtype]
    assert e["max_rel"] <= tol["max_rel"], (tag, e)
    if "max_abs" in tol:
        assert e["max_abs"] <= tol["max_abs"], (tag, e)
    el = float(np.max(np.abs(lse - ref_lse)))
    assert np.all(np.abs(lse - ref_lse) <= lse_bound(dtype, ref_lse)), (tag, "lse", el)
    print(pass_line(tag, shape, e) + f" lse_abs={el:.1e}", flush=True)
    return e


def run_step(inp):
    """The step as a serving engine runs it: the cache's prefix key rows were
    rotated when they were written (done here first), then tv.verify_step
    rotates the queries and the tree's key rows and runs the attention."""
    w = inp["workload"]
    dt = w.kv_dtype
    q_lat = cuda_f32(inp["q_lat"])
    q_rope = cuda_f32(inp["q_rope"])
    c_kv = cuda_cache(inp["c_kv"], dt)
    k_rope = cuda_cache(inp["k_rope"], dt)
    parent = torch.from_numpy(inp["parent"]).cuda()
    P = w.prefix_len
    if P > 0:
        tv.rope_neox_strided(k_rope[:, :P, :], None, w.theta)
    out, lse = tv.verify_step(q_lat, q_rope, c_kv, k_rope, parent, P, w.theta, w.sm_scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse, q_rope, k_rope


def check_rope(got_q, got_k, ref, inp, max_frac=1e-4):
    dt = inp["workload"].kv_dtype
    mp = int(ref["pos_k"].max())
    nq = rope_mismatch(got_q.cpu().numpy(), ref["q_rope"], O.as_f64(inp["q_rope"], "f32"), "f32", mp)
    assert nq[0] == 0 and nq[1] <= max_frac, ("q_rope", nq)
    nk = rope_mismatch(O.as_f64(cache_numpy(got_k, dt), dt), ref["k_rope"], O.as_f64(inp["k_rope"], dt), dt, mp)
    assert nk[0] == 0 and nk[1] <= max_frac, ("k_rope", nk)


SMALL = [n for n in W.WORKLOADS if n != W.SERVING]


@pytest.mark.parametrize("name", SMALL)
def test_step_parity(name):
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w)
    ref = O.verify_step(inp["q_lat"], inp["q_rope"], inp["c_kv"], inp["k_rope"], inp["parent"], w.prefix_len,
                        w.theta, w.sm_scale, w.kv_dtype)
    out, lse, q_rope, k_rope = run_step(inp)
    check_rope(q_rope, k_rope, ref, inp)
    check_out(name, w.describe(), out, lse, ref["out"], ref["lse"], w.kv_dtype)


def test_step_parity_serving_scale():
    """Full serving shape on the GPU, every tree of the batch against the
    oracle."""
    w = W.WORKLOADS[W.SERVING]
    inp = W.make_inputs(w)
    out, lse, q_rope, k_rope = run_step(inp)
    ref = O.verify_step(inp["q_lat"], inp["q_rope"], inp["c_kv"], inp["k_rope"], inp["parent"], w.prefix_len,
                        w.theta, w.sm_scale, w.kv_dtype)
    check_rope(q_rope, k_rope, ref, inp)
    check_out(w.name, w.describe(), out, lse, ref["out"], ref["lse"], w.kv_dtype)


# ---------------------------------------------------------------------------
# Attention alone on oracle-rotated inputs, edge and ragged shapes
# ---------------------------------------------------------------------------
EDGE = [
    # B, H, q_len, prefix, d_c, d_r, dtype, tree
    (1, 1, 1, 0, 64, 32, "f32", "chain"),      # single node, no prefix
    (2, 3, 1, 100, 128, 32, "f32", "chain"),   # autoregressive decode (budget 0)
    (1, 2, 64, 37, 64, 32, "f32", "rrt"),      # largest tree
    (1, 2, 64, 0, 64, 64, "f32", "chain"),     # largest chain, no prefix (causal prefill)
    (1, 1, 1, 5000, 512, 64, "f32", "chain"),  # long prefix, one row: split-kv + merge
    (2, 4, 9, 3001, 512, 64, "f32", "branch4"),
    (3, 5, 7, 1000, 256, 64, "bf16", "rrt"),   # ragged everything
    (2, 4, 64, 200, 512, 64, "bf16", "wide"),
    (1, 16, 33, 300, 512, 64, "bf16", "branch4"),
    (2, 64, 33, 700, 512, 64, "bf16", "branch4"),
    (1, 7, 13, 129, 512, 32, "f32", "rrt"),
    # bf16 cache, d_c = 512, d_r = 64: the matrix-core kernel
    (3, 8, 5, 40, 512, 64, "bf16", "rrt"),        # R = 40: only a partial row block
    (2, 16, 8, 1000, 512, 64, "bf16", "chain"),   # R = 128: exactly one full block
    (1, 1, 1, 0, 512, 64, "bf16", "chain"),       # one row, one key
    (1, 3, 64, 1, 512, 64, "bf16", "rrt"),        # largest tree, 1-row prefix
    (2, 64, 9, 4097, 512, 64, "bf16", "branch4"), # few blocks: every block split
    (5, 32, 17, 333, 512, 64, "bf16", "wide"),    # ragged rows and kv tail
    (1, 128, 33, 100, 512, 64, "bf16", "branch4"),  # 128 heads
    (2, 7, 19, 333, 512, 64, "bf16", "rrt"),       # odd head count: nodes straddle row blocks
    # fp32 cache, d_c = 512, d_r = 64: the fp32 matrix-core kernel
    (3, 1, 256, 0, 512, 64, "f32", "rrt"),        # tree keys only, 4-word masks, 4 row blocks
    (1, 1, 1, 0, 512, 64, "f32", "chain"),        # one row, one key
    (5, 3, 17, 64, 512, 64, "f32", "wide"),       # prefix of exactly two tiles, partial row block
    (2, 64, 33, 700, 512, 64, "f32", "branch4"),  # full 64-row blocks, kv pieces
    (4, 16, 8, 0, 512, 64, "f32", "chain"),       # R = 128: two full blocks, causal prefill
    (3, 64, 44, 40, 512, 64, "f32", "rrt"),       # 132 blocks of 64 rows: the 64-row form by default
    (9, 64, 30, 20, 512, 64, "f32", "branch4"),   # 270 such blocks: the last blocks cut into kv pieces
    (1, 256, 9, 64, 512, 64, "f32", "chain"),     # 256 heads
    (2, 7, 19, 333, 512, 64, "f32", "rrt"),       # odd head count: nodes straddle row blocks
]


def _edge_inputs(B, H, q, P, d_c, d_r, dt, tree, seed):
    rng = np.random.default_rng(seed)
    kv = P + q
    scale = 0.5 if dt == "bf16" else 1.0
    q_lat = (rng.standard_normal((B, q, H, d_c), dtype=np.float32) * scale).astype(np.float32)
    q_rope = (rng.standard_normal((B, q, H, d_r), dtype=np.float32) * scale).astype(np.float32)
    c_kv = (rng.standard_normal((B, kv, d_c), dtype=np.float32) * scale).astype(np.float32)
    k_rope = (rng.standard_normal((B, kv, d_r), dtype=np.float32) * scale).astype(np.float32)
    if dt == "bf16":
        c_kv, k_rope = W.f32_to_bf16_bits(c_kv), W.f32_to_bf16_bits(k_rope)
    parent = np.stack([W.TREES[tree](q, rng) for _ in range(B)]).astype(np.int32)
    return q_lat, q_rope, c_kv, k_rope, parent


@pytest.mark.parametrize("case", EDGE, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}dc{c[4]}dr{c[5]}{c[6]}{c[7]}" for c in EDGE])
def test_attention_edge_shapes(case):
    B, H, q, P, d_c, d_r, dt, tree = case
    q_lat, q_rope, c_kv, k_rope, parent = _edge_inputs(*case, seed=zlib.crc32(str(case).encode()))
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, dt),
                                     O.as_f64(k_rope, dt), parent, P, sm)
    out, lse = tv.verify_attn(cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(c_kv, dt), cuda_cache(k_rope, dt),
                              torch.from_numpy(parent).cuda(), P, sm, return_lse=True)
    torch.cuda.synchronize()
    check_out("edge", str(case), out, lse, ref_out, ref_lse, dt)


# ---------------------------------------------------------------------------
# RoPE and positions alone
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d_r", [32, 64, 128])
def test_rope_bitwise(dt, d_r):
    rng = np.random.default_rng(d_r)
    n_seq, n_tok, n_head = 3, 50, 4
    x = rng.standard_normal((n_seq, n_tok, n_head, d_r), dtype=np.float32)
    if dt == "bf16":
        x = W.f32_to_bf16_bits(x)
    pos = rng.integers(0, 9000, size=(n_seq, n_tok)).astype(np.int32)
    ref = O.rope_neox_stored(O.as_f64(x, dt), pos[:, :, None], 10000.0, dt)
    xt = cuda_cache(x, dt)
    tv.rope_neox_strided(xt, torch.from_numpy(pos).cuda(), 10000.0)
    torch.cuda.synchronize()
    n = rope_mismatch(O.as_f64(cache_numpy(xt, dt), dt), ref, O.as_f64(x, dt), dt, 9000)
    assert n[0] == 0 and n[1] <= 1e-3, n


def test_rope_strided_view_and_default_positions():
    """Rotating a slice of a cache (strided rows) with pos=None uses the row index."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((2, 40, 64), dtype=np.float32)
    kt = cuda_f32(k)
    tv.rope_neox_strided(kt[:, 3:30, :], None, 10000.0)
    torch.cuda.synchronize()
    got = kt.cpu().numpy()
    ref = O.rope_neox_stored(k[:, 3:30].astype(np.float64), np.arange(27)[None, :], 10000.0, "f32")
    assert np.array_equal(got[:, :3], k[:, :3]) and np.array_equal(got[:, 30:], k[:, 30:])
    n = rope_mismatch(got[:, 3:30], ref, k[:, 3:30], "f32", 30)
    assert n[0] == 0 and n[1] <= 1e-3, n


def test_tree_positions_exact():
    rng = np.random.default_rng(6)
    for q in (1, 2, 9, 33, 64):
        parent = np.stack([W.tree_rrt(q, rng), W.tree_chain(q), W.tree_branch(q, rng)]).astype(np.int32)
        got = tv.tree_positions(torch.from_numpy(parent).cuda(), 8192).cpu().numpy()
        assert np.array_equal(got, O.node_positions(parent, 8192))


# ---------------------------------------------------------------------------
# Mask invariants on the GPU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_non_ancestors_bitwise(dt):
    B, H, q, P, d_c, d_r = 2, 8, 17, 300, 512, 64
    q_lat, q_rope, c_kv, k_rope, parent = _edge_inputs(B, H, q, P, d_c, d_r, dt, "rrt", seed=7)
    args = lambda ck, kr: (cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(ck, dt), cuda_cache(kr, dt),
                           torch.from_numpy(parent).cuda(), P, 0.04)
    base = tv.verify_attn(*args(c_kv, k_rope)).cpu().numpy()
    big = W.f32_to_bf16_bits(np.full(d_c, 3.0e4, np.float32)) if dt == "bf16" else np.float32(3.0e4)
    for b in range(B):
        for i in (0, q // 2, q - 1):
            anc = set(O.ancestors_of(parent[b], i))
            ck, kr = c_kv.copy(), k_rope.copy()
            for m in range(q):
                if m not in anc:
                    ck[b, P + m] = big
                    kr[b, P + m] = big if dt == "f32" else big[:d_r]
            got = tv.verify_attn(*args(ck, kr)).cpu().numpy()
            assert np.array_equal(got[b, i], base[b, i]), (b, i)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_constant_latent_and_root_copy(dt):
    B, H, q, P, d_c, d_r = 2, 4, 9, 0, 512, 64
    q_lat, q_rope, c_kv, k_rope, parent = _edge_inputs(B, H, q, P, d_c, d_r, dt, "rrt", seed=8)
    pt = torch.from_numpy(parent).cuda()
    # Root with no prefix sees only its own row: the output is that row exactly.
    out = tv.verify_attn(cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(c_kv, dt), cuda_cache(k_rope, dt), pt, P,
                         0.04).cpu().numpy()
    for b in range(B):
        assert np.array_equal(out[b, 0], np.broadcast_to(O.as_f64(c_kv, dt)[b, 0].astype(np.float32), (H, d_c)))
    # A constant latent of ones gives ones (softmax rows sum to 1).
    ones = np.ones_like(O.as_f64(c_kv, dt), dtype=np.float32)
    ones_c = W.f32_to_bf16_bits(ones) if dt == "bf16" else ones
    out1 = tv.verify_attn(cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(ones_c, dt), cuda_cache(k_rope, dt), pt,
                          P, 0.04).cpu().numpy()
    assert np.max(np.abs(out1 - 1.0)) <= 4 * 2.0 ** -23


def test_bf16_cache_value_range():
    """The default bf16-cache kernel converts the latent (value) rows to fp16:
    exact for magnitudes from 2^-17 to 65504 (smaller ones rounded to fp16's
    2^-24 spacing, at most 2^-25 off).  Latent values with
    magnitudes spread over 2^-24 .. 2^15.5 (both signs; small queries keep the
    scores moderate) must still give the oracle's output."""
    rng = np.random.default_rng(17)
    B, H, q, P, d_c, d_r = 2, 8, 9, 700, 512, 64
    kv = P + q
    mag = np.exp2(rng.uniform(-24.0, 15.5, (B, kv, d_c)))
    c_kv32 = (mag * np.where(rng.random((B, kv, d_c)) < 0.5, -1.0, 1.0)).astype(np.float32)
    c_kv = W.f32_to_bf16_bits(c_kv32)
    k_rope = W.f32_to_bf16_bits((rng.standard_normal((B, kv, d_r)) * 0.5).astype(np.float32))
    q_lat = (rng.standard_normal((B, q, H, d_c)) * 2e-5).astype(np.float32)
    q_rope = (rng.standard_normal((B, q, H, d_r)) * 0.5).astype(np.float32)
    parent = np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, "bf16"),
                                     O.as_f64(k_rope, "bf16"), parent, P, sm)
    out, lse = tv.verify_attn(cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(c_kv, "bf16"), cuda_cache(k_rope, "bf16"),
                              torch.from_numpy(parent).cuda(), P, sm, return_lse=True)
    torch.cuda.synchronize()
    check_out("bf16 latent values 2^-24..2^15.5", "B2 H8 q9 P700", out, lse, ref_out, ref_lse, "bf16")


@pytest.mark.parametrize("rise", [30.0, 100.0])
def test_bf16_late_large_scores_resweep(rise):
    """Scores that rise far above the first tile's max must still give the
    softmax of the oracle: by ~rise log2 units, past the default kernel's
    fp16-weight headroom (2^15) at 30, past the one-term option's (2^64) at
    100; both kernels."""
    rng = np.random.default_rng(91)
    B, H, q, P, d_c, d_r = 1, 4, 3, 300, 512, 64
    kv = P + q
    u = (rng.standard_normal(d_c) * 0.5).astype(np.float32)
    q_lat = np.broadcast_to(u, (B, q, H, d_c)).astype(np.float32).copy()
    q_rope = np.zeros((B, q, H, d_r), np.float32)
    sm = 0.25
    base = rise / (sm * float(u.astype(np.float64) @ u) * np.log2(np.e))
    t = np.zeros(kv, np.float32)
    t[64:] = base * (1.0 + 0.2 * rng.random(kv - 64)).astype(np.float32)
    c_kv32 = (t[:, None] * u[None, :])[None].astype(np.float32)
    c_kv = W.f32_to_bf16_bits(c_kv32)
    k_rope = W.f32_to_bf16_bits(np.zeros((B, kv, d_r), np.float32))
    parent = W.tree_chain(q)[None].astype(np.int32)
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, "bf16"),
                                     O.as_f64(k_rope, "bf16"), parent, P, sm)
    assert ref_lse.min() > (rise - 1.0) * np.log(2.0)  # far above the first tile's max of 0
    args = (cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(c_kv, "bf16"), cuda_cache(k_rope, "bf16"),
            torch.from_numpy(parent).cuda(), P, sm)
    out, lse = tv.verify_attn(*args, return_lse=True)
    torch.cuda.synchronize()
    check_out(f"late-large-scores rise {rise:g}", "B1 H4 q3 P300", out, lse, ref_out, ref_lse, "bf16")
    out, lse = tv.verify_attn_ex(*args, tv.TV_ATTN_BF16_QUERIES, return_lse=True)
    torch.cuda.synchronize()
    check_out(f"late-large-scores rise {rise:g} bf16 queries", "B1 H4 q3 P300", out, lse, ref_out, ref_lse,
              "bf16_queries")


# The attention kernels: (d_c, d_r, cache dtype) that selects each, and the
# tv_verify_attn_ex flags.  The fp32 matrix-core kernel takes these tests'
# small batches on its 32-row form by default; TV_ATTN_F32_WIDE keeps them on
# the 64-row form.
KERNELS = {"mfma_bf16": (512, 64, "bf16"), "mfma_f32": (512, 64, "f32"), "mfma_f32_wide": (512, 64, "f32"),
           "valu": (64, 32, "f32")}
KERNEL_FLAGS = {"mfma_f32_wide": tv.TV_ATTN_F32_WIDE}


def _attn(kernel, *args, **kw):
    return tv.verify_attn_ex(*args, flags=KERNEL_FLAGS.get(kernel, 0), **kw)


def _check_tol(e, dt, tag):
    assert e["max_rel"] <= TOL[dt]["max_rel"], (tag, e)
    if "max_abs" in TOL[dt]:
        assert e["max_abs"] <= TOL[dt]["max_abs"], (tag, e)


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("q", [1, 3])
def test_tree_key_at_every_tile_position(kernel, q):
    """Prefix lengths 28 .. 71 put the first tree key at every position of a
    key tile, in units of one, two and three tiles, with and without kv
    pieces (B = 1 splits the kv range, B = 256 does not), on each kernel.
    The fp32 matrix-core kernel once dropped a visible tree key held in score
    register 0 of a later tile; every case here is checked against the
    oracle.  (Its 32-row form takes B = 1 by default, B = 256 takes the
    64-row form either way.)"""
    d_c, d_r, dt = KERNELS[kernel]
    for B, H in ((1, 16), (256, 4)):
        rng = np.random.default_rng(B + q)
        sc = 0.5 if dt == "bf16" else 1.0
        ql = (rng.standard_normal((B, q, H, d_c), dtype=np.float32) * sc).astype(np.float32)
        qr = (rng.standard_normal((B, q, H, d_r), dtype=np.float32) * sc).astype(np.float32)
        ck_all = (rng.standard_normal((B, 71 + q, d_c), dtype=np.float32) * sc).astype(np.float32)
        kr_all = (rng.standard_normal((B, 71 + q, d_r), dtype=np.float32) * sc).astype(np.float32)
        if dt == "bf16":
            ck_all, kr_all = W.f32_to_bf16_bits(ck_all), W.f32_to_bf16_bits(kr_all)
        par = np.stack([W.tree_chain(q) for _ in range(B)]).astype(np.int32)
        args = (cuda_f32(ql), cuda_f32(qr))
        rows = [0, B - 1]
        for P in range(28, 72):
            ck = np.ascontiguousarray(ck_all[:, :P + q])
            kr = np.ascontiguousarray(kr_all[:, :P + q])
            out = _attn(kernel, *args, cuda_cache(ck, dt), cuda_cache(kr, dt), torch.from_numpy(par).cuda(), P,
                        0.04).cpu().numpy()
            ref, _ = O.verify_attn(ql[rows].astype(np.float64), qr[rows].astype(np.float64),
                                   O.as_f64(ck[rows], dt), O.as_f64(kr[rows], dt), par[rows], P, 0.04)
            _check_tol(errors(out[rows], ref), dt, (kernel, B, P, q))


def _depths(parent_row):
    d = [0] * len(parent_row)
    for i in range(1, len(parent_row)):
        d[i] = d[parent_row[i]] + 1
    return d


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("P", [0, 37, 1000])
def test_zero_queries_give_visible_mean(kernel, P):
    """Zero queries make every visible score 0: each output row is the plain
    mean of the latent rows the node sees -- the whole prefix, its ancestors
    and itself, P + depth + 1 rows -- and lse = ln(P + depth + 1).  Checked
    against that closed form (float64 sums of the stored rows, depths by a
    walk written here), tightly: the weights are exactly 1 in every kernel,
    so only float32 summation order separates the two."""
    d_c, d_r, dt = KERNELS[kernel]
    B, H, q = 3, 8, 17
    _, _, c_kv, k_rope, parent = _edge_inputs(B, H, q, P, d_c, d_r, dt, "branch4", seed=40 + P)
    z_lat = np.zeros((B, q, H, d_c), np.float32)
    z_rope = np.zeros((B, q, H, d_r), np.float32)
    out, lse = _attn(kernel, cuda_f32(z_lat), cuda_f32(z_rope), cuda_cache(c_kv, dt), cuda_cache(k_rope, dt),
                     torch.from_numpy(parent).cuda(), P, 0.04, return_lse=True)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    C = O.as_f64(c_kv, dt)
    want = np.zeros((B, q, d_c))
    cnt = np.zeros((B, q))
    for b in range(B):
        dep = _depths(parent[b])
        pre = C[b, :P].sum(axis=0)
        for i in range(q):
            rows, n = [], i
            while n != -1:
                rows.append(P + n)
                n = int(parent[b, n])
            assert len(rows) == dep[i] + 1
            cnt[b, i] = P + dep[i] + 1
            want[b, i] = (pre + C[b, rows].sum(axis=0)) / cnt[b, i]
    e = errors(out, np.broadcast_to(want[:, :, None, :], out.shape))
    assert e["max_rel"] <= 1e-5 and e["max_abs"] <= 1e-5, (kernel, P, e)
    assert np.abs(lse - np.log(cnt)[:, :, None]).max() <= 2e-6 * np.log(cnt.max() + 1), (kernel, P)


def _topological_relabel(parent_row, rng):
    """A random relabelling of the nodes that keeps parents before children
    and the root at 0: returns (new label of each node, relabelled parents)."""
    q = len(parent_row)
    kids = [[] for _ in range(q)]
    for i in range(1, q):
        kids[parent_row[i]].append(i)
    order, ready = [0], list(kids[0])
    while ready:
        n = ready.pop(int(rng.integers(0, len(ready))))
        order.append(n)
        ready += kids[n]
    new = np.empty(q, np.int64)
    new[order] = np.arange(q)
    newp = np.full(q, -1, np.int32)
    for i in range(1, q):
        newp[new[i]] = new[parent_row[i]]
    assert all(0 <= newp[i] < i for i in range(1, q))
    return new, newp


@pytest.mark.parametrize("kernel", list(KERNELS))
def test_topological_relabelling_permutes_outputs(kernel):
    """Relabelling a tree into another topological order (moving each node's
    query rows and latent/rope row with it) permutes the outputs: node i's
    result comes back at its new label.  Scores and weights of a (row, key)
    pair are the same numbers either way; only the order of the float32
    accumulation over the tree keys changes, so the two results agree to
    1e-5 (and each matches the oracle)."""
    d_c, d_r, dt = KERNELS[kernel]
    B, H, q, P = 2, 8, 33, 300
    rng = np.random.default_rng(55)
    q_lat, q_rope, c_kv, k_rope, parent = _edge_inputs(B, H, q, P, d_c, d_r, dt, "rrt", seed=56)
    ql2, qr2, ck2, kr2, par2 = q_lat.copy(), q_rope.copy(), c_kv.copy(), k_rope.copy(), parent.copy()
    news = []
    for b in range(B):
        new, newp = _topological_relabel(parent[b], rng)
        news.append(new)
        par2[b] = newp
        ql2[b, new] = q_lat[b]
        qr2[b, new] = q_rope[b]
        ck2[b, P + new] = c_kv[b, P:]
        kr2[b, P + new] = k_rope[b, P:]
    run = lambda a, bq, c, k, p: _attn(kernel, cuda_f32(a), cuda_f32(bq), cuda_cache(c, dt), cuda_cache(k, dt),
                                       torch.from_numpy(p).cuda(), P, 0.04).cpu().numpy()
    o1, o2 = run(q_lat, q_rope, c_kv, k_rope, parent), run(ql2, qr2, ck2, kr2, par2)
    back = np.stack([o2[b, news[b]] for b in range(B)])
    e = errors(back, o1)
    assert e["max_rel"] <= 1e-5, (kernel, e)
    ref, _ = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, dt),
                           O.as_f64(k_rope, dt), parent, P, 0.04)
    _check_tol(errors(o1, ref), dt, kernel)


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("rise", [80.0, 150.0])
def test_f32_late_large_scores_resweep(rise, wide):
    """fp32 cache: scores that rise far above the first tile's max a few tiles
    into a unit must still give the oracle's softmax: by ~80 log2 units (past
    the fp32 kernel's 64-unit headroom, so the unit sweeps again) and by ~150
    (where weights against the first tile's max would overflow fp32).
    1 x 64 heads x 33 nodes gives both forms units of several tiles (the
    32-row form: 3 kv pieces of 128 keys, halves of four 16-key tiles); the
    rise comes at key 40, inside the first half of the first piece, so that
    half and the 64-row form's first unit sweep again."""
    rng = np.random.default_rng(92)
    B, H, q, P, d_c, d_r = 1, 64, 33, 300, 512, 64
    kv = P + q
    u = (rng.standard_normal(d_c) * 0.5).astype(np.float32)
    q_lat = np.broadcast_to(u, (B, q, H, d_c)).astype(np.float32).copy()
    q_rope = np.zeros((B, q, H, d_r), np.float32)
    sm = 0.25
    base = rise / (sm * float(u.astype(np.float64) @ u) * np.log2(np.e))
    t = np.zeros(kv, np.float32)
    t[40:] = base * (1.0 + 0.2 * rng.random(kv - 40)).astype(np.float32)
    c_kv = (t[:, None] * u[None, :])[None].astype(np.float32)
    k_rope = np.zeros((B, kv, d_r), np.float32)
    parent = W.tree_chain(q)[None].astype(np.int32)
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, "f32"),
                                     O.as_f64(k_rope, "f32"), parent, P, sm)
    assert ref_lse.min() > (rise - 1.0) * np.log(2.0)
    out, lse = tv.verify_attn_ex(cuda_f32(q_lat), cuda_f32(q_rope), cuda_f32(c_kv), cuda_f32(k_rope),
                                 torch.from_numpy(parent).cuda(), P, sm, tv.TV_ATTN_F32_WIDE if wide else 0,
                                 return_lse=True)
    torch.cuda.synchronize()
    check_out(f"f32 late-large-scores rise {rise:g} {'64-row' if wide else '32-row'}", "B1 H64 q33 P300", out, lse,
              ref_out, ref_lse, "f32")


def test_f32_row_block_and_piece_edges():
    """fp32 cache at 512/64, both forms: row counts on either side of the
    32- and 64-row blocks (R = 31 .. 97 with one head) over prefixes that
    give the 32-row form's units an odd or even number of 16-key tiles, one
    tile, or a half with no keys, each against the oracle."""
    sm = float(np.float32(1.0 / np.sqrt(576.0)))
    for q in (31, 32, 33, 63, 64, 65, 95, 97):
        for P in (0, 5, 300, 1000):
            B, H = 2, 1
            seed = 7000 + 10 * q + P
            q_lat, q_rope, c_kv, k_rope, parent = _edge_inputs(B, H, q, P, 512, 64, "f32", "rrt", seed=seed)
            ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, "f32"),
                                             O.as_f64(k_rope, "f32"), parent, P, sm)
            args = (cuda_f32(q_lat), cuda_f32(q_rope), cuda_f32(c_kv), cuda_f32(k_rope),
                    torch.from_numpy(parent).cuda(), P, sm)
            for flags in (0, tv.TV_ATTN_F32_WIDE):
                out, lse = tv.verify_attn_ex(*args, flags, return_lse=True)
                check_out(f"f32 edges flags={flags}", f"B{B} H{H} q{q} P{P}", out, lse, ref_out, ref_lse, "f32")


# ---------------------------------------------------------------------------
# The fp32 kernel's 64-row form on the small shapes (TV_ATTN_F32_WIDE)
# ---------------------------------------------------------------------------
F32_EDGE = [c for c in EDGE if c[4:7] == (512, 64, "f32")]


@pytest.mark.parametrize("case", F32_EDGE, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}{c[7]}" for c in F32_EDGE])
def test_f32_wide_edge_shapes(case):
    """The fp32-cache edge shapes on the 64-row form, against the oracle and
    against the default (32-row) form: the same fp32 products, summed in
    another order where a unit's keys are cut differently."""
    B, H, q, P, d_c, d_r, dt, kind = case
    q_lat, q_rope, c_kv, k_rope, parent = _edge_inputs(B, H, q, P, d_c, d_r, dt, kind, seed=B * 1000 + q)
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, dt),
                                     O.as_f64(k_rope, dt), parent, P, sm)
    args = (cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(c_kv, dt), cuda_cache(k_rope, dt),
            torch.from_numpy(parent).cuda(), P, sm)
    out, lse = tv.verify_attn_ex(*args, tv.TV_ATTN_F32_WIDE, return_lse=True)
    out0, lse0 = tv.verify_attn(*args, return_lse=True)
    out, lse, out0, lse0 = (t.cpu().numpy() for t in (out, lse, out0, lse0))
    check_out("edge-wide", str(case), torch.from_numpy(out), torch.from_numpy(lse), ref_out, ref_lse, dt)
    e = errors(out, out0)
    assert e["max_abs"] <= 1e-5 and e["max_rel"] <= 1e-2, (case, e)
    assert np.abs(lse - lse0).max() <= 4e-5, case


# ---------------------------------------------------------------------------
# The bf16-queries option (tv_verify_attn_ex, TV_ATTN_BF16_QUERIES)
# ---------------------------------------------------------------------------
BF16Q_EDGE = [c for c in EDGE if c[4:7] == (512, 64, "bf16")]


@pytest.mark.parametrize("case", BF16Q_EDGE, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}{c[7]}" for c in BF16Q_EDGE])
def test_bf16_queries_edge_shapes(case):
    """The one-term query kernel on the bf16-cache edge shapes, against the
    oracle at the bf16 bound."""
    B, H, q, P, d_c, d_r, dt, tree = case
    q_lat, q_rope, c_kv, k_rope, parent = _edge_inputs(*case, seed=zlib.crc32(str(case).encode()))
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, dt),
                                     O.as_f64(k_rope, dt), parent, P, sm)
    out, lse = tv.verify_attn_ex(cuda_f32(q_lat), cuda_f32(q_rope), cuda_cache(c_kv, dt), cuda_cache(k_rope, dt),
                                 torch.from_numpy(parent).cuda(), P, sm, tv.TV_ATTN_BF16_QUERIES, return_lse=True)
    torch.cuda.synchronize()
    check_out("edge bf16 queries", str(case), out, lse, ref_out, ref_lse, "bf16_queries")


def test_bf16_queries_serving_scale():
    """The serving batch through the one-term query kernel (rotated by the
    step's RoPE first), every tree against the oracle."""
    w = W.WORKLOADS[W.SERVING]
    inp = W.make_inputs(w)
    ref = O.verify_step(inp["q_lat"], inp["q_rope"], inp["c_kv"], inp["k_rope"], inp["parent"], w.prefix_len,
                        w.theta, w.sm_scale, w.kv_dtype)
    q_lat, q_rope = cuda_f32(inp["q_lat"]), cuda_f32(inp["q_rope"])
    c_kv, k_rope = cuda_cache(inp["c_kv"], "bf16"), cuda_cache(inp["k_rope"], "bf16")
    parent = torch.from_numpy(inp["parent"]).cuda()
    tv.rope_neox_strided(k_rope[:, :w.prefix_len, :], None, w.theta)
    tv.tree_rope(q_rope, k_rope, parent, w.prefix_len, w.theta)
    out, lse = tv.verify_attn_ex(q_lat, q_rope, c_kv, k_rope, parent, w.prefix_len, w.sm_scale,
                                 tv.TV_ATTN_BF16_QUERIES, return_lse=True)
    torch.cuda.synchronize()
    check_out(w.name + " bf16 queries", w.describe(), out, lse, ref["out"], ref["lse"], "bf16_queries")


@pytest.mark.parametrize("d_r,H,dt", [(6, 3, "f32"), (32, 8, "bf16"), (64, 64, "bf16"), (128, 1, "f32"),
                                      (64, 600, "f32"), (2, 5, "bf16")])
def test_tree_rope_shapes(d_r, H, dt):
    """tv_tree_rope on its own over row widths and head counts that take each
    path of the kernel (whole 16-byte items, one pair at a time, more items
    than a workgroup prefetches, several nodes per workgroup): query rows and
    the tree's key rows turn at prefix + depth like the oracle's rotation;
    the prefix key rows are untouched."""
    rng = np.random.default_rng(d_r * 1000 + H)
    B, q, P = 3, 33, 50
    qr = rng.standard_normal((B, q, H, d_r), dtype=np.float32)
    kr = rng.standard_normal((B, P + q, d_r), dtype=np.float32)
    if dt == "bf16":
        kr = W.f32_to_bf16_bits(kr)
    parent = np.stack([W.tree_rrt(q, rng) for _ in range(B)]).astype(np.int32)
    qt, kt = cuda_f32(qr), cuda_cache(kr, dt)
    tv.tree_rope(qt, kt, torch.from_numpy(parent).cuda(), P, 10000.0)
    torch.cuda.synchronize()
    pos_q = O.node_positions(parent, P)
    ref_q = O.rope_neox_stored(O.as_f64(qr, "f32"), pos_q[:, :, None], 10000.0, "f32")
    ref_k = O.rope_neox_stored(O.as_f64(kr, dt)[:, P:], pos_q, 10000.0, dt)
    got_k = O.as_f64(cache_numpy(kt, dt), dt)
    mp = int(pos_q.max())
    nq = rope_mismatch(qt.cpu().numpy(), ref_q, O.as_f64(qr, "f32"), "f32", mp)
    nk = rope_mismatch(got_k[:, P:], ref_k, O.as_f64(kr, dt)[:, P:], dt, mp)
    assert nq[0] == 0 and nq[1] <= 1e-3 and nk[0] == 0 and nk[1] <= 1e-3, (nq, nk)
    assert np.array_equal(got_k[:, :P], O.as_f64(kr, dt)[:, :P])
