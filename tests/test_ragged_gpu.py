"""Ragged batches (tv_verify_attn_ragged): requests with their own prefix length
and tree size in one launch, lengths in device memory.  Each request's rows are
compared with the float64 oracle run on that request alone."""
import zlib

import numpy as np
import pytest
import torch

from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W
from tvcompare import errors, lse_bound

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-5, max_rel=1e-2), "bf16": dict(max_rel=2e-2)}


def _ragged_inputs(q_lens, prefixes, H, d_c, d_r, dt, stride_pad, seed):
    rng = np.random.default_rng(seed)
    B = len(q_lens)
    S = max(p + q for p, q in zip(prefixes, q_lens)) + stride_pad
    N = sum(q_lens)
    scale = 0.5 if dt == "bf16" else 1.0
    q_lat = (rng.standard_normal((N, H, d_c), dtype=np.float32) * scale).astype(np.float32)
    q_rope = (rng.standard_normal((N, H, d_r), dtype=np.float32) * scale).astype(np.float32)
    c_kv = (rng.standard_normal((B, S, d_c), dtype=np.float32) * scale).astype(np.float32)
    k_rope = (rng.standard_normal((B, S, d_r), dtype=np.float32) * scale).astype(np.float32)
    if dt == "bf16":
        c_kv, k_rope = W.f32_to_bf16_bits(c_kv), W.f32_to_bf16_bits(k_rope)
    trees = ["rrt", "chain", "wide", "branch4"]
    parent = np.concatenate([W.TREES[trees[b % 4]](q, rng) for b, q in enumerate(q_lens) if q > 0] or
                            [np.zeros(0, np.int64)]).astype(np.int32)
    return q_lat, q_rope, c_kv, k_rope, parent


def _cache(a, dt):
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(q_lens, prefixes, H, d_c, d_r, dt, max_q=None, stride_pad=0):
    tag = f"ragged q={q_lens} P={prefixes} H={H} d_c={d_c} {dt}"
    print(tag, flush=True)
    max_q = max_q or max(max(q_lens), 1)
    q_lat, q_rope, c_kv, k_rope, parent = _ragged_inputs(q_lens, prefixes, H, d_c, d_r, dt, stride_pad,
                                                         seed=zlib.crc32(tag.encode()))
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    out, lse = tv.verify_attn_ragged(torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(),
                                     _cache(c_kv, dt), _cache(k_rope, dt), torch.from_numpy(parent).cuda(),
                                     torch.tensor(prefixes, dtype=torch.int32).cuda(),
                                     torch.tensor(q_lens, dtype=torch.int32).cuda(), max_q, sm, return_lse=True)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    s = 0
    for b, (q, P) in enumerate(zip(q_lens, prefixes)):
        if q == 0:
            continue
        kv = P + q
        ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat[None, s:s + q], "f32"), O.as_f64(q_rope[None, s:s + q], "f32"),
                                         O.as_f64(c_kv[b:b + 1, :kv], dt), O.as_f64(k_rope[b:b + 1, :kv], dt),
                                         parent[None, s:s + q], P, sm)
        e = errors(out[s:s + q], ref_out[0])
        assert e["max_rel"] <= TOL[dt]["max_rel"], (tag, b, e)
        if "max_abs" in TOL[dt]:
            assert e["max_abs"] <= TOL[dt]["max_abs"], (tag, b, e)
        assert np.all(np.abs(lse[s:s + q] - ref_lse[0]) <= lse_bound(dt, ref_lse[0])), (tag, b)
        s += q


CASES = [
    # q_len per request, prefix per request, H, d_c, d_r, dtype
    ([5, 33, 1, 64, 17], [100, 0, 3000, 511, 8192], 8, 512, 64, "bf16"),
    ([0, 9, 0, 33], [50, 200, 0, 1000], 16, 512, 64, "bf16"),       # empty requests
    ([33, 33], [100000, 100], 16, 512, 64, "bf16"),                   # one long request: its own kv pieces
    ([1, 7, 65, 200], [0, 40, 129, 5], 3, 64, 32, "f32"),             # VALU kernel, multi-word trees
    ([130, 2, 256], [7000, 1, 300], 2, 512, 64, "f32"),
    ([0, 9, 0, 33], [50, 200, 0, 1000], 16, 512, 64, "f32"),         # empty requests, the fp32 32-row form
    ([33] * 6, [900, 40, 2500, 0, 64, 1500], 64, 512, 64, "f32"),    # the fp32 64-row form (6 x 33 blocks)
    ([3, 1], [0, 0], 1, 128, 64, "bf16"),                              # no prefix at all
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_ragged(case):
    _check(*case)


def test_ragged_many_requests():
    rng = np.random.default_rng(8)
    B = 40
    q_lens = [int(x) for x in rng.integers(0, 65, size=B)]
    prefixes = [int(x) for x in rng.integers(0, 4000, size=B)]
    _check(q_lens, prefixes, 16, 512, 64, "bf16", stride_pad=17)


def test_ragged_bound_above_lengths():
    """max_q_len and the cache stride above every request's use."""
    _check([9, 20], [300, 64], 8, 512, 64, "bf16", max_q=200, stride_pad=5000)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_equal_lengths_match_uniform(dt):
    """Every request the same size: the ragged call and tv_verify_attn agree.
    The two plan their kv pieces independently, and the bf16 kernel rounds
    each weight relative to its piece's reference max, so with the bf16 cache
    they agree to the bf16 bound (each also against the oracle); with the
    fp32 cache only the order of float32 sums differs."""
    B, q, P, H = 3, 17, 700, 8
    d_c, d_r = (512, 64) if dt == "bf16" else (256, 64)
    q_lat, q_rope, c_kv, k_rope, parent = _ragged_inputs([q] * B, [P] * B, H, d_c, d_r, dt, 0, seed=9)
    sm = 0.0417
    args = [torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(c_kv, dt), _cache(k_rope, dt)]
    r = tv.verify_attn_ragged(*args, torch.from_numpy(parent).cuda(), torch.full((B,), P, dtype=torch.int32).cuda(),
                              torch.full((B,), q, dtype=torch.int32).cuda(), q, sm)
    u = tv.verify_attn(args[0].view(B, q, H, d_c), args[1].view(B, q, H, d_r), args[2], args[3],
                       torch.from_numpy(parent.reshape(B, q)).cuda(), P, sm)
    torch.cuda.synchronize()
    r, u = r.cpu().numpy().reshape(B, q, H, d_c), u.cpu().numpy()
    e = errors(r, u)
    assert e["max_rel"] <= (1e-5 if dt == "f32" else TOL["bf16"]["max_rel"]), e
    ref, _ = O.verify_attn(O.as_f64(q_lat.reshape(B, q, H, d_c), "f32"), O.as_f64(q_rope.reshape(B, q, H, d_r), "f32"),
                           O.as_f64(c_kv, dt), O.as_f64(k_rope, dt), parent.reshape(B, q), P, sm)
    for got in (r, u):
        assert errors(got, ref)["max_rel"] <= TOL[dt]["max_rel"]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_step(dt):
    """RoPE at prefix_len[b] + depth for each request, then the attention,
    against the oracle's whole step on each request alone."""
    q_lens, prefixes, H = [17, 0, 33, 5, 70], [300, 10, 4096, 0, 1000], 4
    d_c, d_r = (512, 64) if dt == "bf16" else (128, 32)
    theta = 10000.0
    q_lat, q_rope, c_kv, k_rope, parent = _ragged_inputs(q_lens, prefixes, H, d_c, d_r, dt, 7, seed=31)
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    kr = _cache(k_rope, dt)
    for b, P in enumerate(prefixes):  # the cache's prefix rows were rotated when written
        if P:
            tv.rope_neox_strided(kr[b:b + 1, :P, :], None, theta)
    qr = torch.from_numpy(q_rope).cuda()
    out, lse = tv.verify_step_ragged(torch.from_numpy(q_lat).cuda(), qr, _cache(c_kv, dt), kr,
                                     torch.from_numpy(parent).cuda(), torch.tensor(prefixes, dtype=torch.int32).cuda(),
                                     torch.tensor(q_lens, dtype=torch.int32).cuda(), max(q_lens), theta, sm,
                                     return_lse=True)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    s = 0
    for b, (q, P) in enumerate(zip(q_lens, prefixes)):
        if q == 0:
            continue
        kv = P + q
        ref = O.verify_step(q_lat[None, s:s + q], q_rope[None, s:s + q], c_kv[b:b + 1, :kv], k_rope[b:b + 1, :kv],
                            parent[None, s:s + q], P, theta, sm, dt)
        e = errors(out[s:s + q], ref["out"][0])
        assert e["max_rel"] <= TOL[dt]["max_rel"], (b, e)
        s += q


def test_ragged_many_row_blocks_tail_pieces():
    """Enough row blocks to fill the GPU: full row blocks stay whole and each
    request's partial last block is cut into pieces on the device."""
    rng = np.random.default_rng(12)
    B = 20
    q_lens = [int(x) for x in rng.integers(17, 65, size=B)]
    prefixes = [int(x) for x in rng.integers(100, 3000, size=B)]
    _check(q_lens, prefixes, 64, 512, 64, "bf16")


@pytest.mark.parametrize("which", ["bench_like", "uniform", "few_long", "many_short", "valu", "f32_mfma",
                                   "f32_mfma_wide"])
def test_ragged_records_match_plan_model(which):
    """The prep kernel's records (plan choice, class order, numbering) equal
    the host model's word for word, and the attention over them matches the
    oracle on sampled requests."""
    import ragged_plan_model as RP
    rng = np.random.default_rng(zlib.crc32(which.encode()))
    dt, H, d_c, d_r = "bf16", 16, 512, 64
    if which == "bench_like":
        q_lens = [int(x) for x in rng.choice([9, 17, 33], 32)]
        prefixes = [int(x) for x in rng.integers(2048, 16384, 32)]
    elif which == "uniform":
        q_lens, prefixes = [33] * 16, [3000] * 16
    elif which == "few_long":
        q_lens, prefixes = [33, 5, 40], [30000, 45000, 12000]
    elif which == "many_short":
        q_lens = [int(x) for x in rng.integers(0, 20, 150)]
        prefixes = [int(x) for x in rng.integers(0, 600, 150)]
    elif which == "valu":
        dt, H, d_c, d_r = "f32", 4, 128, 32
        q_lens = [int(x) for x in rng.integers(1, 70, 12)]
        prefixes = [int(x) for x in rng.integers(0, 9000, 12)]
    elif which == "f32_mfma":  # the fp32 kernel's 32-row form (10 x 9 blocks of 64 rows at most)
        dt, H, d_c, d_r = "f32", 8, 512, 64
        q_lens = [int(x) for x in rng.integers(1, 70, 10)]
        prefixes = [int(x) for x in rng.integers(0, 5000, 10)]
    else:  # its 64-row form (6 x 33 blocks of 64 rows at most)
        dt, H, d_c, d_r = "f32", 64, 512, 64
        q_lens = [int(x) for x in rng.integers(9, 34, 6)]
        prefixes = [int(x) for x in rng.integers(0, 1500, 6)]
    max_q = max(q_lens)
    print(f"ragged records {which} B={len(q_lens)}", flush=True)
    q_lat, q_rope, c_kv, k_rope, parent = _ragged_inputs(q_lens, prefixes, H, d_c, d_r, dt, 5, seed=1)
    S = c_kv.shape[1]
    ws_n = tv.load().tv_verify_attn_ragged_workspace_size(len(q_lens), H, max_q, S, d_c, d_r,
                                                          tv.TV_BF16 if dt == "bf16" else tv.TV_F32)
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda")
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    out = tv.verify_attn_ragged(torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(c_kv, dt),
                                _cache(k_rope, dt), torch.from_numpy(parent).cuda(),
                                torch.tensor(prefixes, dtype=torch.int32).cuda(),
                                torch.tensor(q_lens, dtype=torch.int32).cuda(), max_q, sm, workspace=ws)
    torch.cuda.synchronize()
    if d_c == 512 and d_r == 64:  # the matrix-core kernels: rows per workgroup, workgroups at once, costs
        if dt == "bf16":
            rpb, target, cost = 64, 256, RP.COST_DEFAULT
        else:  # the 32-row form when the bound has at most 128 blocks of 64 rows
            narrow = len(q_lens) * -(-(max_q * H) // 64) <= 128
            assert narrow == (which == "f32_mfma")
            rpb, target, cost = (32 if narrow else 64), 256, RP.COST_F32
    else:
        rpb, target, cost = 16, 512, RP.COST_DEFAULT
    model = RP.records_words(RP.plan(prefixes, q_lens, H, max_q, S, rpb, target, cost))
    got = ws[:4 * len(model)].view(torch.int32).cpu().numpy().tolist()
    assert got == model
    out = out.cpu().numpy()
    starts = np.cumsum([0] + q_lens)
    for b in rng.choice(len(q_lens), size=min(3, len(q_lens)), replace=False):
        q, P, s = q_lens[b], prefixes[b], starts[b]
        if q == 0:
            continue
        ref, _ = O.verify_attn(O.as_f64(q_lat[None, s:s + q], "f32"), O.as_f64(q_rope[None, s:s + q], "f32"),
                               O.as_f64(c_kv[b:b + 1, :P + q], dt), O.as_f64(k_rope[b:b + 1, :P + q], dt),
                               parent[None, s:s + q], P, sm)
        e = errors(out[s:s + q], ref[0])
        assert e["max_rel"] <= TOL[dt]["max_rel"], (which, b, e)


def test_ragged_records_unsorted_large_batch():
    """More than 2048 requests: the prep kernel keeps request order (no sort
    in LDS); its records still equal the model's and every sampled request
    matches the oracle."""
    import ragged_plan_model as RP
    rng = np.random.default_rng(2100)
    B, H, d_c, d_r = 2100, 2, 512, 64
    q_lens = [int(x) for x in rng.integers(0, 6, B)]
    prefixes = [int(x) for x in rng.integers(0, 100, B)]
    print(f"ragged unsorted B={B}", flush=True)
    q_lat, q_rope, c_kv, k_rope, parent = _ragged_inputs(q_lens, prefixes, H, d_c, d_r, "bf16", 0, seed=4)
    S = c_kv.shape[1]
    ws_n = tv.load().tv_verify_attn_ragged_workspace_size(B, H, max(q_lens), S, d_c, d_r, tv.TV_BF16)
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda")
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    out = tv.verify_attn_ragged(torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(c_kv, "bf16"),
                                _cache(k_rope, "bf16"), torch.from_numpy(parent).cuda(),
                                torch.tensor(prefixes, dtype=torch.int32).cuda(),
                                torch.tensor(q_lens, dtype=torch.int32).cuda(), max(q_lens), sm, workspace=ws)
    torch.cuda.synchronize()
    model = RP.plan(prefixes, q_lens, H, max(q_lens), S, 64, 256)
    assert model["cls_id"] == list(range(2 * B))
    words = RP.records_words(model)
    assert ws[:4 * len(words)].view(torch.int32).cpu().numpy().tolist() == words
    out = out.cpu().numpy()
    starts = np.cumsum([0] + q_lens)
    for b in rng.choice(B, size=12, replace=False):
        q, P, s = q_lens[b], prefixes[b], starts[b]
        if q == 0:
            continue
        ref, _ = O.verify_attn(O.as_f64(q_lat[None, s:s + q], "f32"), O.as_f64(q_rope[None, s:s + q], "f32"),
                               O.as_f64(c_kv[b:b + 1, :P + q], "bf16"), O.as_f64(k_rope[b:b + 1, :P + q], "bf16"),
                               parent[None, s:s + q], P, sm)
        assert errors(out[s:s + q], ref[0])["max_rel"] <= TOL["bf16"]["max_rel"], b


@pytest.mark.parametrize("step", [False, True])
def test_ragged_lengths_past_node_rows(step):
    """Device lengths that sum past the caller's rows (n_nodes, the rows of
    q_lat): the request crossing n_nodes keeps its first nodes, later requests
    none.  The buffers carry guard rows past n_nodes, so even an unclamped run
    would stay inside them; the guard rows must come back untouched, and the
    rows below n_nodes must match the oracle on the clamped requests.  The
    records equal the host model's word for word."""
    import ragged_plan_model as RP
    dt, H, d_c, d_r = "bf16", 8, 512, 64
    q_lens, prefixes = [17, 33, 20, 9], [300, 1200, 40, 5000]
    N, G = 40, 24                       # request 1 keeps 23 of its 33 nodes; 2 and 3 none
    theta = 10000.0
    print(f"ragged node bound step={step}", flush=True)
    q_lat, q_rope, c_kv, k_rope, parent = _ragged_inputs(q_lens, prefixes, H, d_c, d_r, dt, 3, seed=77)
    assert q_lat.shape[0] == sum(q_lens) >= N + G
    ql_full = torch.from_numpy(q_lat[:N + G]).cuda()
    qr_full = torch.from_numpy(q_rope[:N + G].copy()).cuda()
    par_full = torch.from_numpy(parent[:N + G]).cuda()
    out_full = torch.full((N + G, H, d_c), 7.0, dtype=torch.float32, device="cuda")
    lse_full = torch.full((N + G, H), 7.0, dtype=torch.float32, device="cuda")
    kr = _cache(k_rope, dt)
    if step:  # the cache's prefix rows were rotated when written
        for b, P in enumerate(prefixes):
            tv.rope_neox_strided(kr[b:b + 1, :P, :], None, theta)
    k_before = kr.clone()
    S = c_kv.shape[1]
    ws_n = tv.load().tv_verify_attn_ragged_workspace_size(len(q_lens), H, max(q_lens), S, d_c, d_r, tv.TV_BF16)
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda")
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    pl = torch.tensor(prefixes, dtype=torch.int32).cuda()
    qlt = torch.tensor(q_lens, dtype=torch.int32).cuda()
    args = (ql_full[:N], qr_full[:N], _cache(c_kv, dt), kr, par_full[:N], pl, qlt, max(q_lens))
    if step:
        tv.verify_step_ragged(*args, theta, sm, out=out_full[:N], lse=lse_full[:N], workspace=ws)
    else:
        tv.verify_attn_ragged(*args, sm, out=out_full[:N], lse=lse_full[:N], workspace=ws)
    torch.cuda.synchronize()
    model = RP.plan(prefixes, q_lens, H, max(q_lens), S, 64, 256, n_nodes=N)
    assert [r["q_len"] for r in model["req"]] == [17, 23, 0, 0]
    words = RP.records_words(model)
    assert ws[:4 * len(words)].view(torch.int32).cpu().numpy().tolist() == words
    out, lse = out_full.cpu().numpy(), lse_full.cpu().numpy()
    assert np.all(out[N:] == 7.0) and np.all(lse[N:] == 7.0)
    assert np.array_equal(qr_full[N:].cpu().numpy(), q_rope[N:N + G])
    kb, ka = k_before.view(torch.int16).cpu().numpy(), kr.view(torch.int16).cpu().numpy()
    for b, (qk, P) in enumerate(zip([17, 23, 0, 0], prefixes)):
        # rows past the kept nodes (and every prefix row) are never rotated
        assert np.array_equal(ka[b, :P], kb[b, :P]) and np.array_equal(ka[b, P + qk:], kb[b, P + qk:]), b
    s = 0
    for b, (q, P) in enumerate(zip([17, 23], prefixes)):
        kv = P + q
        if step:
            ref = O.verify_step(q_lat[None, s:s + q], q_rope[None, s:s + q], c_kv[b:b + 1, :kv],
                                k_rope[b:b + 1, :kv], parent[None, s:s + q], P, theta, sm, dt)
            ref_out, ref_lse = ref["out"], ref["lse"]
        else:
            ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat[None, s:s + q], "f32"),
                                             O.as_f64(q_rope[None, s:s + q], "f32"), O.as_f64(c_kv[b:b + 1, :kv], dt),
                                             O.as_f64(k_rope[b:b + 1, :kv], dt), parent[None, s:s + q], P, sm)
        e = errors(out[s:s + q], ref_out[0])
        assert e["max_rel"] <= TOL[dt]["max_rel"], (b, e)
        assert np.all(np.abs(lse[s:s + q] - ref_lse[0]) <= lse_bound(dt, ref_lse[0])), b
        s += q
