"""GPU parity for the steps after verify: greedy tokens (tv_argmax_rows), greedy
tree accept (tv_tree_accept) and compaction (tv_kv_compact), through the C ABI,
against the CPU oracle.  Integer and byte results: bit-exact."""
import numpy as np
import pytest
import torch

from oracle import accept_oracle as A
from tree_verify_mla_tv_amd import tv
from tree_verify_mla_tv_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _bf16_to_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("vocab", [1, 3, 7, 8, 64, 1000, 4099, 32768])
def test_argmax_rows_exact(dtype, vocab):
    rng = np.random.default_rng(vocab)
    rows = rng.integers(-4, 5, size=(37, vocab)).astype(np.float32)   # many ties
    rows[1] = rng.standard_normal(vocab).astype(np.float32)
    if vocab > 2:
        rows[2, vocab // 2] = np.nan
        rows[2, vocab - 1] = np.nan
        rows[3, :] = -np.inf
        rows[4, :] = 0.0
        rows[4, 1] = -0.0
        rows[5, vocab - 1] = np.inf
        rows[6, :] = -0.0
        rows[6, vocab - 1] = 0.0
    if dtype == "bf16":
        bits = W.f32_to_bf16_bits(rows)
        want = A.greedy_tokens(_bf16_to_f64(bits))
        got = tv.argmax_rows(_bf16(bits))
    else:
        want = A.greedy_tokens(rows)
        got = tv.argmax_rows(torch.from_numpy(rows).to(DEV))
    assert got.cpu().numpy().tolist() == want.tolist()


def test_argmax_rows_unaligned_rows_take_scalar_path():
    rng = np.random.default_rng(5)
    buf = rng.standard_normal(7 * 10 + 1).astype(np.float32)
    t = torch.from_numpy(buf).to(DEV)[1:].view(7, 10)   # 4-byte aligned, not 16
    want = A.greedy_tokens(buf[1:].reshape(7, 10))
    assert tv.argmax_rows(t.contiguous() if not t.is_contiguous() else t).cpu().numpy().tolist() == want.tolist()


def _trees(rng, B, q, shape):
    return np.stack([W.TREES[shape](q, rng) for _ in range(B)]).astype(np.int32)


@pytest.mark.parametrize("shape", ["rrt", "chain", "wide", "branch4"])
@pytest.mark.parametrize("q", [1, 2, 9, 33, 64])
def test_tree_accept_exact(shape, q):
    rng = np.random.default_rng(q * 7 + len(shape))
    B = 23
    par = _trees(rng, B, q, shape)
    # Small token alphabet: many matches, duplicate siblings included.
    draft = rng.integers(0, 3, size=(B, q)).astype(np.int32)
    target = rng.integers(0, 3, size=(B, q)).astype(np.int32)
    path, n, bonus = A.tree_accept(par, draft, target)
    g = [torch.from_numpy(x).to(DEV) for x in (par, draft, target)]
    gp, gn, gb = tv.tree_accept(*g)
    assert gp.cpu().numpy().tolist() == path.tolist()
    assert gn.cpu().numpy().tolist() == n.tolist()
    assert gb.cpu().numpy().tolist() == bonus.tolist()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_compact_exact(dtype):
    rng = np.random.default_rng(11)
    B, P, q, dc, dr = 9, 37, 33, 512, 64
    kv = P + q + 5                                    # rows past the tree must stay
    par = _trees(rng, B, q, "branch4")
    draft = rng.integers(0, 2, size=(B, q)).astype(np.int32)
    target = rng.integers(0, 2, size=(B, q)).astype(np.int32)
    path, n, _ = A.tree_accept(par, draft, target)
    c = rng.standard_normal((B, kv, dc)).astype(np.float32)
    r = rng.standard_normal((B, kv, dr)).astype(np.float32)
    if dtype == "bf16":
        cb, rb = W.f32_to_bf16_bits(c), W.f32_to_bf16_bits(r)
        want_c, want_r = A.kv_compact(cb, rb, path, n, P)
        gc, gr = _bf16(cb), _bf16(rb)
    else:
        want_c, want_r = A.kv_compact(c, r, path, n, P)
        gc, gr = torch.from_numpy(c).to(DEV), torch.from_numpy(r).to(DEV)
    tv.kv_compact(gc, gr, torch.from_numpy(path.astype(np.int32)).to(DEV),
                  torch.from_numpy(n.astype(np.int32)).to(DEV), P)
    if dtype == "bf16":
        got_c = gc.view(torch.int16).cpu().numpy().view(np.uint16)
        got_r = gr.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got_c, got_r = gc.cpu().numpy(), gr.cpu().numpy()
    assert np.array_equal(got_c, want_c) and np.array_equal(got_r, want_r)
    assert n.max() > 0 and n.min() >= 0


def test_accept_step_end_to_end_serving_shape():
    """Greedy tokens -> accept -> compaction at the serving shape (B=32, q=33,
    K2-class vocabulary, bf16 cache), all on the GPU, against the oracle."""
    w = W.WORKLOADS[W.SERVING]
    rng = np.random.default_rng(42)
    par = np.stack([W.tree_branch(w.q_len, rng) for _ in range(w.B)]).astype(np.int32)
    x = W.make_accept_inputs(par, W.SERVE_VOCAB, seed=43)
    target = A.greedy_tokens(x["logits"])
    path, n, bonus = A.tree_accept(par, x["draft"], target)
    assert np.array_equal(n, x["depth"])
    g_logits = torch.from_numpy(x["logits"]).to(DEV)
    g_target = tv.argmax_rows(g_logits)
    assert g_target.cpu().numpy().tolist() == target.tolist()
    gp, gn, gb = tv.tree_accept(torch.from_numpy(par).to(DEV), torch.from_numpy(x["draft"]).to(DEV), g_target)
    assert gp.cpu().numpy().tolist() == path.tolist() and gn.cpu().numpy().tolist() == n.tolist()
    assert gb.cpu().numpy().tolist() == bonus.tolist()
    # Compaction on a smaller-prefix cache of the same row shape.
    P = 300
    c = W.f32_to_bf16_bits(rng.standard_normal((w.B, P + w.q_len, w.d_c)).astype(np.float32))
    r = W.f32_to_bf16_bits(rng.standard_normal((w.B, P + w.q_len, w.d_r)).astype(np.float32))
    want_c, want_r = A.kv_compact(c, r, path, n, P)
    gc, gr = _bf16(c), _bf16(r)
    tv.kv_compact(gc, gr, gp, gn, P)
    assert np.array_equal(gc.view(torch.int16).cpu().numpy().view(np.uint16), want_c)
    assert np.array_equal(gr.view(torch.int16).cpu().numpy().view(np.uint16), want_r)
