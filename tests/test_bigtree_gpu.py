"""Trees of more than 64 nodes (several 64-bit ancestor words per node), up to
256: verify attention on both kernels, the whole step, tree positions, greedy
accept and compaction, against the CPU oracles."""
import zlib

import numpy as np
import pytest
import torch

from oracle import accept_oracle as A
from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W
from tvcompare import errors, lse_bound

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-5, max_rel=1e-2), "bf16": dict(max_rel=2e-2)}


def _inputs(B, H, q, P, d_c, d_r, dt, tree, seed):
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


def _cache(a, dt):
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


CASES = [
    # B, H, q, P, d_c, d_r, dtype, tree
    (2, 4, 65, 37, 512, 64, "bf16", "rrt"),
    (1, 8, 100, 0, 512, 64, "bf16", "chain"),     # causal prefill of 100 tokens
    (2, 2, 128, 1000, 512, 64, "bf16", "wide"),
    (1, 4, 200, 4096, 512, 64, "bf16", "branch4"),
    (1, 3, 256, 1, 512, 64, "bf16", "rrt"),
    (1, 16, 256, 8192, 512, 64, "bf16", "branch4"),
    (2, 3, 65, 5, 64, 32, "f32", "rrt"),
    (1, 2, 130, 700, 128, 64, "f32", "chain"),
    (1, 4, 256, 300, 512, 64, "f32", "branch4"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}dc{c[4]}{c[6]}{c[7]}" for c in CASES])
def test_attention_big_trees(case):
    B, H, q, P, d_c, d_r, dt, tree = case
    print(f"big tree attention {case}", flush=True)
    q_lat, q_rope, c_kv, k_rope, parent = _inputs(*case, seed=zlib.crc32(str(case).encode()))
    sm = float(np.float32(1.0 / np.sqrt(d_c + d_r)))
    out, lse = tv.verify_attn(torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(c_kv, dt),
                              _cache(k_rope, dt), torch.from_numpy(parent).cuda(), P, sm, return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = O.verify_attn(O.as_f64(q_lat, "f32"), O.as_f64(q_rope, "f32"), O.as_f64(c_kv, dt),
                                     O.as_f64(k_rope, dt), parent, P, sm)
    e = errors(out.cpu().numpy(), ref_out)
    assert e["max_rel"] <= TOL[dt]["max_rel"], e
    if "max_abs" in TOL[dt]:
        assert e["max_abs"] <= TOL[dt]["max_abs"], e
    assert np.all(np.abs(lse.cpu().numpy() - ref_lse) <= lse_bound(dt, ref_lse))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_non_ancestors_bitwise_big_tree(dt):
    """Perturbing the rows of tree nodes that are not ancestors of node i
    leaves row i of the output bit-identical (words 2 and 3 of the masks)."""
    B, H, q, P, d_c, d_r = 1, 4, 230, 100, 512, 64
    q_lat, q_rope, c_kv, k_rope, parent = _inputs(B, H, q, P, d_c, d_r, dt, "rrt", seed=21)
    args = lambda ck, kr: (torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_rope).cuda(), _cache(ck, dt),
                           _cache(kr, dt), torch.from_numpy(parent).cuda(), P, 0.04)
    base = tv.verify_attn(*args(c_kv, k_rope)).cpu().numpy()
    big = W.f32_to_bf16_bits(np.full(d_c, 3.0e4, np.float32)) if dt == "bf16" else np.float32(3.0e4)
    for i in (0, 70, 150, q - 1):
        anc = set(O.ancestors_of(parent[0], i))
        ck = c_kv.copy()
        for m in range(q):
            if m not in anc:
                ck[0, P + m] = big
        got = tv.verify_attn(*args(ck, k_rope)).cpu().numpy()
        assert np.array_equal(got[0, i], base[0, i]), i


def test_step_and_positions_big_tree():
    B, H, q, P = 2, 4, 129, 513
    rng = np.random.default_rng(3)
    parent = np.stack([W.tree_branch(q, rng), W.tree_rrt(q, rng)]).astype(np.int32)
    got = tv.tree_positions(torch.from_numpy(parent).cuda(), P).cpu().numpy()
    assert np.array_equal(got, O.node_positions(parent, P))
    q_lat, q_rope, c_kv, k_rope, _ = _inputs(B, H, q, P, 512, 64, "bf16", "chain", seed=4)
    theta, sm = 10000.0, float(np.float32(1.0 / np.sqrt(576)))
    kr = _cache(k_rope, "bf16")
    tv.rope_neox_strided(kr[:, :P, :], None, theta)
    qr = torch.from_numpy(q_rope).cuda()
    out, lse = tv.verify_step(torch.from_numpy(q_lat).cuda(), qr, _cache(c_kv, "bf16"), kr,
                              torch.from_numpy(parent).cuda(), P, theta, sm, return_lse=True)
    torch.cuda.synchronize()
    ref = O.verify_step(q_lat, q_rope, c_kv, k_rope, parent, P, theta, sm, "bf16")
    e = errors(out.cpu().numpy(), ref["out"])
    assert e["max_rel"] <= 2e-2, e


@pytest.mark.parametrize("q", [65, 128, 256])
def test_accept_and_compact_big_tree(q):
    rng = np.random.default_rng(q)
    B, vocab = 5, 512
    parent = np.stack([W.tree_branch(q, rng, max_children=2) for _ in range(B)]).astype(np.int32)
    x = W.make_accept_inputs(parent, vocab, seed=q, max_accept=q)
    target = A.greedy_tokens(x["logits"]).astype(np.int32)
    path, n, bonus = tv.tree_accept(torch.from_numpy(parent).cuda(), torch.from_numpy(x["draft"]).cuda(),
                                    torch.from_numpy(target).cuda())
    r_path, r_n, r_bonus = A.tree_accept(parent, x["draft"], target)
    assert np.array_equal(path.cpu().numpy(), r_path) and np.array_equal(n.cpu().numpy(), r_n)
    assert np.array_equal(bonus.cpu().numpy(), r_bonus)
    P, d_c, d_r = 40, 512, 64
    c_kv = W.f32_to_bf16_bits(rng.standard_normal((B, P + q, d_c), dtype=np.float32))
    k_rope = W.f32_to_bf16_bits(rng.standard_normal((B, P + q, d_r), dtype=np.float32))
    c_t, k_t = _cache(c_kv, "bf16"), _cache(k_rope, "bf16")
    tv.kv_compact(c_t, k_t, path, n, P)
    r_c, r_k = A.kv_compact(c_kv, k_rope, r_path, r_n, P)
    assert np.array_equal(c_t.view(torch.int16).cpu().numpy().view(np.uint16), r_c)
    assert np.array_equal(k_t.view(torch.int16).cpu().numpy().view(np.uint16), r_k)


def test_accept_deep_chain():
    """A chain of 256 whose draft tokens all match: the walk crosses every
    group of 64 nodes and accepts 255."""
    q, B = 256, 2
    parent = np.stack([W.tree_chain(q) for _ in range(B)]).astype(np.int32)
    draft = np.arange(B * q, dtype=np.int32).reshape(B, q) % 1000
    target = np.roll(draft, -1, axis=1)
    target[:, -1] = 7
    target[1, 150] = 999999  # tree 1 stops after node 150
    path, n, bonus = tv.tree_accept(torch.from_numpy(parent).cuda(), torch.from_numpy(draft).cuda(),
                                    torch.from_numpy(target).cuda())
    r_path, r_n, r_bonus = A.tree_accept(parent, draft, target)
    assert list(r_n) == [255, 150]
    assert np.array_equal(path.cpu().numpy(), r_path) and np.array_equal(n.cpu().numpy(), r_n)
    assert np.array_equal(bonus.cpu().numpy(), r_bonus)
