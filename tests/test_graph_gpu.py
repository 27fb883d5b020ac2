"""The verify calls captured in a HIP graph (torch.cuda.CUDAGraph): every
replay, with new inputs written eagerly in between, equals an eager call on the
same inputs bit for bit.  The ragged graph is replayed with different
per-request lengths each time: its launch sizes come from the bounds and the
plan is made on the device, so one captured graph serves every batch within
them."""
import numpy as np
import pytest
import torch

from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(W.f32_to_bf16_bits(a)).view(np.int16)).cuda().view(torch.bfloat16)


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_uniform_graph_replays(dt):
    rng = np.random.default_rng(11)
    B, H, q, P, d_c, d_r = 4, 16, 17, 700, 512, 64
    parent = torch.from_numpy(np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)).cuda()
    q_lat = torch.empty(B, q, H, d_c, device="cuda")
    q_rope = torch.empty(B, q, H, d_r, device="cuda")
    if dt == "bf16":
        c_kv = torch.empty(B, P + q, d_c, device="cuda", dtype=torch.bfloat16)
        k_rope = torch.empty(B, P + q, d_r, device="cuda", dtype=torch.bfloat16)
    else:
        c_kv = torch.empty(B, P + q, d_c, device="cuda")
        k_rope = torch.empty(B, P + q, d_r, device="cuda")
    code = tv.TV_BF16 if dt == "bf16" else tv.TV_F32
    ws_n = max(tv.workspace_size(B, H, q, P, d_c, d_r, code), 1)
    ws_g = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    out_g, out_e = torch.empty_like(q_lat), torch.empty_like(q_lat)
    lse_g, lse_e = torch.empty(B, q, H, device="cuda"), torch.empty(B, q, H, device="cuda")
    call = lambda out, lse, ws: tv.verify_attn(q_lat, q_rope, c_kv, k_rope, parent, P, 0.04, out=out, lse=lse,
                                                workspace=ws)

    def fill(seed):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        for t in (q_lat, q_rope, c_kv, k_rope):
            t.copy_(torch.randn(t.shape, device="cuda", generator=g) * 0.5)

    fill(0)
    graph = _capture(lambda: call(out_g, lse_g, ws_g))
    for rep in range(4):
        fill(100 + rep)
        graph.replay()
        torch.cuda.synchronize()
        call(out_e, lse_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), rep


def test_ragged_graph_replays_with_new_lengths():
    rng = np.random.default_rng(12)
    B, H, max_q, S, d_c, d_r = 12, 16, 33, 6000, 512, 64
    N = B * max_q
    q_lat = torch.empty(N, H, d_c, device="cuda")
    q_rope = torch.empty(N, H, d_r, device="cuda")
    c_kv = _bf16(rng.standard_normal((B, S, d_c), dtype=np.float32) * 0.5)
    k_rope = _bf16(rng.standard_normal((B, S, d_r), dtype=np.float32) * 0.5)
    parent = torch.empty(N, dtype=torch.int32, device="cuda")
    pl = torch.empty(B, dtype=torch.int32, device="cuda")
    ql = torch.empty(B, dtype=torch.int32, device="cuda")
    ws_n = tv.load().tv_verify_attn_ragged_workspace_size(B, H, max_q, S, d_c, d_r, tv.TV_BF16)
    ws_g = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    out_g, out_e = torch.zeros_like(q_lat), torch.zeros_like(q_lat)
    call = lambda out, ws: tv.verify_attn_ragged(q_lat, q_rope, c_kv, k_rope, parent, pl, ql, max_q, 0.04, out=out,
                                                 workspace=ws)

    def fill(seed):
        r = np.random.default_rng(seed)
        q_lens = [int(x) for x in r.integers(0, max_q + 1, B)]
        prefixes = [int(x) for x in r.integers(0, S - max_q, B)]
        pars = [W.tree_branch(q, r).astype(np.int32) for q in q_lens if q > 0]
        packed = np.concatenate(pars) if pars else np.zeros(0, np.int32)
        par = np.zeros(N, np.int32)
        par[:len(packed)] = packed
        parent.copy_(torch.from_numpy(par))
        pl.copy_(torch.tensor(prefixes, dtype=torch.int32))
        ql.copy_(torch.tensor(q_lens, dtype=torch.int32))
        q_lat.copy_(torch.from_numpy(r.standard_normal((N, H, d_c), dtype=np.float32)))
        q_rope.copy_(torch.from_numpy(r.standard_normal((N, H, d_r), dtype=np.float32)))
        return sum(q_lens)

    fill(0)
    graph = _capture(lambda: call(out_g, ws_g))
    for rep in range(4):
        n = fill(200 + rep)
        graph.replay()
        torch.cuda.synchronize()
        call(out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g[:n], out_e[:n]), rep


def test_ragged_step_graph_replays():
    """The whole ragged step (tree RoPE in place, then attention) captured
    once; before each replay and each eager call the caches and queries are
    restored, so every replay must equal the eager step: output, rotated
    queries and rotated tree key rows."""
    rng = np.random.default_rng(13)
    B, H, max_q, S, d_c, d_r = 6, 16, 17, 3000, 512, 64
    N = B * max_q
    q_lat = torch.empty(N, H, d_c, device="cuda")
    q_rope = torch.empty(N, H, d_r, device="cuda")
    c_kv = _bf16(rng.standard_normal((B, S, d_c), dtype=np.float32) * 0.5)
    k_rope = _bf16(rng.standard_normal((B, S, d_r), dtype=np.float32) * 0.5)
    k0 = k_rope.clone()
    parent = torch.empty(N, dtype=torch.int32, device="cuda")
    pl = torch.empty(B, dtype=torch.int32, device="cuda")
    ql = torch.empty(B, dtype=torch.int32, device="cuda")
    ws_n = tv.load().tv_verify_attn_ragged_workspace_size(B, H, max_q, S, d_c, d_r, tv.TV_BF16)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    out = torch.zeros_like(q_lat)
    step = lambda: tv.verify_step_ragged(q_lat, q_rope, c_kv, k_rope, parent, pl, ql, max_q, 10000.0, 0.04, out=out,
                                         workspace=ws)

    def fill(seed):
        r = np.random.default_rng(seed)
        q_lens = [int(x) for x in r.integers(1, max_q + 1, B)]
        pars = np.concatenate([W.tree_branch(q, r).astype(np.int32) for q in q_lens])
        par = np.zeros(N, np.int32)
        par[:len(pars)] = pars
        parent.copy_(torch.from_numpy(par))
        pl.copy_(torch.tensor([int(x) for x in r.integers(0, S - max_q, B)], dtype=torch.int32))
        ql.copy_(torch.tensor(q_lens, dtype=torch.int32))
        q_lat.copy_(torch.from_numpy(r.standard_normal((N, H, d_c), dtype=np.float32)))
        q_rope.copy_(torch.from_numpy(r.standard_normal((N, H, d_r), dtype=np.float32)))
        k_rope.copy_(k0)
        return sum(q_lens)

    fill(0)
    graph = _capture(step)
    for rep in range(3):
        n = fill(300 + rep)
        graph.replay()
        torch.cuda.synchronize()
        got = (out[:n].clone(), q_rope[:n].clone(), k_rope.clone())
        fill(300 + rep)
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], out[:n]) and torch.equal(got[1], q_rope[:n]) and torch.equal(got[2], k_rope), rep
        assert not torch.equal(k_rope, k0), rep  # the tree key rows were rotated
