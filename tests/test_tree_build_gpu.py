"""GPU parity for the best-first tree builder (tv_tree_build through the C ABI)
against the CPU oracle: parents, tokens, depths, node counts bit-exact, scores
bitwise equal (both sides add in float32 in the same order)."""
import numpy as np
import pytest
import torch

from oracle.tree_build_oracle import best_first_tree
from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(logp, tok, root, budget):
    print(f"tree_build B={logp.shape[0]} D={logp.shape[1]} K={logp.shape[2]} budget={budget}", flush=True)
    out = tv.tree_build(torch.from_numpy(np.ascontiguousarray(logp, dtype=np.float32)).to(DEV),
                        torch.from_numpy(np.ascontiguousarray(tok, dtype=np.int32)).to(DEV),
                        torch.from_numpy(np.ascontiguousarray(root, dtype=np.int32)).to(DEV), budget)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _check(logp, tok, root, budget):
    g_par, g_tok, g_dep, g_sc, g_n = _run(logp, tok, root, budget)
    r_par, r_tok, r_dep, r_sc, r_n = best_first_tree(logp, tok, root, budget)
    np.testing.assert_array_equal(g_n, r_n)
    np.testing.assert_array_equal(g_par, r_par)
    np.testing.assert_array_equal(g_dep, r_dep)
    np.testing.assert_array_equal(g_tok, r_tok)
    np.testing.assert_array_equal(g_sc.view(np.uint32), r_sc.astype(np.float32).view(np.uint32))
    return g_par, g_n


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_serving_shape(seed):
    x = W.make_build_inputs(32, W.BUILD_DEPTH, W.BUILD_TOPK, seed)
    par, n = _check(x["logp"], x["cand_tok"], x["root_tok"], 32)
    assert (n == 32).all()


@pytest.mark.parametrize("B,D,K,budget,sort,alpha", [
    (7, 16, 8, 32, False, 0.3),     # unsorted proposals
    (5, 40, 64, 63, False, 1.0),    # widest K, largest budget
    (5, 63, 2, 63, True, 0.1),      # deep and narrow
    (9, 1, 64, 63, False, 0.5),     # a star
    (9, 1, 5, 63, True, 0.5),       # a star that runs out of candidates
    (6, 20, 1, 13, True, 0.5),      # a chain
    (6, 200, 3, 5, False, 0.5),     # depth far past the budget
    (4, 2, 2, 10, True, 0.5),       # frontier exhausted after 6 nodes
    (3, 8, 4, 0, True, 0.5),        # no draft nodes
    (3, 8, 4, 1, False, 0.5),
    (1000, 12, 6, 40, False, 0.3),  # many requests
    (3, 300, 4, 255, False, 0.3),   # largest budget: four frontier slots per lane
    (2, 128, 64, 255, False, 1.0),  # most ranked candidates (128 depths x 64)
    (4, 255, 1, 255, True, 0.5),    # a 255-node chain
    (3, 1, 64, 255, False, 0.5),    # a star that runs out at 64
    (5, 40, 3, 100, True, 0.2),
])
def test_shapes(B, D, K, budget, sort, alpha):
    x = W.make_build_inputs(B, D, K, seed=B * 7 + D + K, sort=sort, alpha=alpha)
    _check(x["logp"], x["cand_tok"], x["root_tok"], budget)


@pytest.mark.parametrize("value", [0.0, -1.0, -0.0])
def test_all_tied(value):
    B, D, K = 3, 10, 3
    lp = np.full((B, D, K), value, dtype=np.float32)
    tok = np.arange(B * D * K, dtype=np.int32).reshape(B, D, K)
    par, n = _check(lp, tok, np.array([1, 2, 3]), 63)
    assert list(par[0, 1:8]) == [0, 0, 0, 1, 1, 1, 2]  # breadth-first


def test_all_tied_largest_budget():
    """255 draft nodes, every log-prob equal: the breadth-first numbering of
    the complete ternary tree, across all four frontier slots of each lane."""
    B, D, K = 2, 12, 3
    lp = np.zeros((B, D, K), dtype=np.float32)
    tok = np.arange(B * D * K, dtype=np.int32).reshape(B, D, K)
    par, n = _check(lp, tok, np.array([5, 6]), 255)
    assert (n == 255).all()
    assert all(par[0, i] == (i - 1) // K for i in range(1, 256))


def test_nan_inf_and_integer_ties():
    rng = np.random.default_rng(11)
    B, D, K = 16, 10, 12
    lp = rng.integers(-5, 1, size=(B, D, K)).astype(np.float32)
    lp[rng.random((B, D, K)) < 0.1] = np.nan
    lp[rng.random((B, D, K)) < 0.1] = -np.inf
    lp[0] = -np.inf
    lp[1, :, :] = np.nan
    tok = rng.integers(0, 163840, size=(B, D, K)).astype(np.int32)
    _check(lp, tok, rng.integers(0, 100, size=B), 63)


def test_float32_rounding_ties():
    """Sibling log-probs far below the parent score's ulp: whole groups of
    nodes tie after float32 rounding, so the order rests on depth, parent and
    log-prob rank."""
    rng = np.random.default_rng(12)
    B, D, K = 8, 12, 6
    lp = np.empty((B, D, K), dtype=np.float32)
    lp[:, 0, :] = -1.0
    lp[:, 1:, :] = -rng.uniform(1e-9, 4e-8, size=(B, D - 1, K)).astype(np.float32)
    tok = rng.integers(0, 1000, size=(B, D, K)).astype(np.int32)
    _check(lp, tok, np.zeros(B), 63)


def test_built_tree_feeds_verify():
    """The builder's parents are a valid tree for the verify attention (nodes
    in topological order), and the attention over it matches the oracle."""
    x = W.make_build_inputs(2, 8, 4, seed=3)
    par, n = _check(x["logp"], x["cand_tok"], x["root_tok"], 16)
    parent = par.astype(np.int32)
    O.validate_tree(parent)
    rng = np.random.default_rng(4)
    B, q, H, P, dc, dr = 2, 17, 4, 40, 64, 32
    q_lat = rng.standard_normal((B, q, H, dc)).astype(np.float32)
    q_rope = rng.standard_normal((B, q, H, dr)).astype(np.float32)
    c_kv = rng.standard_normal((B, P + q, dc)).astype(np.float32)
    k_rope = rng.standard_normal((B, P + q, dr)).astype(np.float32)
    scale = 1.0 / np.sqrt(dc + dr)
    g = tv.verify_attn(torch.from_numpy(q_lat).to(DEV), torch.from_numpy(q_rope).to(DEV),
                       torch.from_numpy(c_kv).to(DEV), torch.from_numpy(k_rope).to(DEV),
                       torch.from_numpy(parent).to(DEV), P, scale)
    torch.cuda.synchronize()
    ref, _ = O.verify_attn(q_lat.astype(np.float64), q_rope.astype(np.float64), c_kv.astype(np.float64),
                           k_rope.astype(np.float64), parent, P, scale)
    assert np.abs(g.cpu().numpy() - ref).max() < 1e-5
