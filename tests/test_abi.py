"""The C ABI on the host: library loads, exports what include/tv.h declares,
and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

from tree_verify_mla_tv_amd import tv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tv.h")

INV, UNS, OK = tv.TV_ERR_INVALID, tv.TV_ERR_UNSUPPORTED, tv.TV_OK
A = 0x10000  # an aligned, never-dereferenced address: every case below fails validation first


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("tv_rope_neox", "tv_verify_attn", "tv_verify_attn_workspace_size", "tv_status_str",
              "tv_tree_positions", "tv_verify_step", "tv_tree_rope", "tv_argmax_rows", "tv_tree_accept",
              "tv_kv_compact"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = tv.load()
    for s in declared_symbols():
        assert hasattr(lib, s), s
        assert s in tv.SIGNATURES, f"binding lacks {s}"


def test_status_strings():
    assert tv.status_str(OK) == "TV_OK"
    assert "invalid" in tv.status_str(INV)
    assert "not supported" in tv.status_str(UNS)
    assert "launch" in tv.status_str(tv.TV_ERR_LAUNCH)
    assert tv.status_str(99) == "TV_ERR_UNKNOWN"


def _attn(lib, **kw):
    a = dict(q_lat=A, q_rope=A, c_kv=A, k_rope=A, parent=A, prefix=4, B=1, H=2, q=3, d_c=64, d_r=32, dt=0,
             scale=0.1, out=A, lse=None, ws=None, ws_n=0)
    a.update(kw)
    return lib.tv_verify_attn(a["q_lat"], a["q_rope"], a["c_kv"], a["k_rope"], a["parent"], a["prefix"], a["B"],
                              a["H"], a["q"], a["d_c"], a["d_r"], a["dt"], a["scale"], a["out"], a["lse"],
                              a["ws"], a["ws_n"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q_lat=None), INV), (dict(q_rope=None), INV), (dict(c_kv=None), INV), (dict(k_rope=None), INV),
    (dict(parent=None), INV), (dict(out=None), INV),
    (dict(B=0), INV), (dict(H=0), INV), (dict(q=0), INV), (dict(prefix=-1), INV),
    (dict(q=257), UNS), (dict(d_r=33), INV), (dict(d_c=100), UNS), (dict(d_r=16), UNS), (dict(dt=7), INV),
    (dict(q_lat=A + 8), INV), (dict(c_kv=A + 4), INV), (dict(out=A + 12), INV), (dict(parent=A + 2), INV),
    (dict(lse=A + 1), INV), (dict(scale=float("inf")), INV), (dict(scale=float("nan")), INV),
    (dict(prefix=2**31 - 10), INV),
    # one tree's latent rows at 2^31 bytes: bf16 at kv_len 2^21, f32 at 2^20
    (dict(prefix=2**21 - 3, d_c=512, dt=1), UNS), (dict(prefix=2**20 - 3, d_c=512, dt=0), UNS),
])
def test_verify_attn_rejects_before_launch(kw, code):
    assert _attn(tv.load(), **kw) == code


def test_workspace_too_small_is_rejected():
    lib = tv.load()
    # A long prefix with few rows is cut into kv splits, which need workspace.
    need = tv.workspace_size(1, 1, 1, 5000, 512, 64, tv.TV_F32)
    assert need > 0
    assert _attn(lib, B=1, H=1, q=1, prefix=5000, d_c=512, d_r=64, ws=None, ws_n=0) == INV
    assert _attn(lib, B=1, H=1, q=1, prefix=5000, d_c=512, d_r=64, ws=A, ws_n=need - 1) == INV
    assert _attn(lib, B=1, H=1, q=1, prefix=5000, d_c=512, d_r=64, ws=A + 8, ws_n=need) == INV


def test_workspace_size_is_a_function_of_shapes():
    f = tv.workspace_size
    assert f(2, 64, 9, 512, 512, 64, tv.TV_F32) == f(2, 64, 9, 512, 512, 64, tv.TV_F32)
    assert f(1, 1, 1, 5000, 512, 64, tv.TV_F32) > 0
    assert f(0, 1, 1, 10, 512, 64, tv.TV_F32) == 0          # invalid shape -> 0
    assert f(1, 1, 257, 10, 512, 64, tv.TV_F32) == 0         # unsupported -> 0


def test_rope_rejects_before_launch():
    """tv_rope_neox(x, dtype, pos, n_tok, n_head, d_r, tok_stride, theta, stream)."""
    r = tv.load().tv_rope_neox
    assert r(A, 0, None, 0, 1, 64, 64, 1e4, None) == OK                  # nothing to do
    assert r(None, 0, None, 5, 1, 64, 64, 1e4, None) == INV
    assert r(A, 0, None, -1, 1, 64, 64, 1e4, None) == INV
    assert r(A, 0, None, 5, 1, 63, 64, 1e4, None) == INV                  # odd d_r
    assert r(A, 0, None, 5, 1, 256, 256, 1e4, None) == UNS                # d_r > 128
    assert r(A, 0, None, 5, 0, 64, 64, 1e4, None) == INV
    assert r(A, 0, None, 5, 1, 64, -1, 1e4, None) == INV                  # negative stride
    assert r(A, 0, None, 5, 1, 64, 64, 0.0, None) == INV
    assert r(A, 0, None, 5, 1, 64, 64, float("nan"), None) == INV
    assert r(A, 2, None, 5, 1, 64, 64, 1e4, None) == INV                  # dtype
    assert r(A + 4, 0, None, 5, 1, 64, 64, 1e4, None) == INV              # x not 16-byte aligned
    assert r(A, 0, A + 2, 5, 1, 64, 64, 1e4, None) == INV                 # pos not 4-byte aligned
    assert r(A, 0, None, 2**36, 64, 64, 4096, 1e4, None) == UNS           # 2^47 pairs: above the launch limit


def test_rope_strided_rejects_before_launch():
    r = tv.load().tv_rope_neox_strided
    assert r(A, 0, None, 0, 5, 1, 64, 0, 64, 0, 1e4, None) == OK          # nothing to do
    assert r(A, 0, None, 3, 0, 1, 64, 0, 64, 0, 1e4, None) == OK
    assert r(None, 0, None, 1, 5, 1, 64, 0, 64, 0, 1e4, None) == INV
    assert r(A, 0, None, 1, 5, 1, 63, 0, 64, 0, 1e4, None) == INV
    assert r(A, 0, None, 1, 5, 1, 256, 0, 256, 0, 1e4, None) == UNS
    assert r(A, 0, None, 1, 5, 0, 64, 0, 64, 0, 1e4, None) == INV
    assert r(A, 0, None, 1, 5, 1, 64, 0, 64, 0, 0.0, None) == INV
    assert r(A, 0, None, 1, 5, 1, 64, 0, 64, 0, float("nan"), None) == INV
    assert r(A, 2, None, 1, 5, 1, 64, 0, 64, 0, 1e4, None) == INV
    assert r(A + 4, 0, None, 1, 5, 1, 64, 0, 64, 0, 1e4, None) == INV
    assert r(A, 0, A + 2, 1, 5, 1, 64, 0, 64, 0, 1e4, None) == INV


def test_rope_signature_matches_the_specified_boundary():
    """The specified call: tv_rope_neox(x, dtype, pos, int64 n_tok, n_head,
    d_r, int64 tok_stride, theta, stream) -- nine arguments, the token count
    and stride 64-bit."""
    import re as _re
    text = open(HEADER).read()
    m = _re.search(r"tv_status_t tv_rope_neox\((.*?)\);", text, flags=_re.S)
    args = [a.strip() for a in m.group(1).split(",")]
    assert [a.split()[-1].lstrip("*") for a in args] == ["x", "dtype", "pos", "n_tok", "n_head", "d_r", "tok_stride",
                                                         "theta", "stream"]
    assert args[3].startswith("int64_t") and args[6].startswith("int64_t")


def test_tree_positions_rejects_before_launch():
    lib = tv.load()
    assert lib.tv_tree_positions(None, 1, 3, 0, A, None) == INV
    assert lib.tv_tree_positions(A, 1, 3, 0, None, None) == INV
    assert lib.tv_tree_positions(A, 0, 3, 0, A, None) == INV
    assert lib.tv_tree_positions(A, 1, 257, 0, A, None) == UNS
    assert lib.tv_tree_positions(A, 1, 3, -2, A, None) == INV


def test_verify_step_rejects_before_launch():
    lib = tv.load()
    s = lib.tv_verify_step
    assert s(A, A, A, A, A, 4, 1, 2, 3, 64, 32, 0, 0.0, 0.1, A, None, None, 0, None) == INV   # theta
    assert s(A, A, A, A, A, 4, 1, 2, 257, 64, 32, 0, 1e4, 0.1, A, None, None, 0, None) == UNS  # q_len
    assert s(A, None, A, A, A, 4, 1, 2, 3, 64, 32, 0, 1e4, 0.1, A, None, None, 0, None) == INV


def test_tree_rope_rejects_before_launch():
    r = tv.load().tv_tree_rope
    assert r(A, A, 0, A, 4, 1, 2, 3, 64, 0.0, None) == INV      # theta
    assert r(A, A, 0, A, 4, 1, 2, 257, 64, 1e4, None) == UNS     # q_len
    assert r(A, A, 3, A, 4, 1, 2, 3, 64, 1e4, None) == INV      # dtype
    assert r(A, A, 0, A, 4, 1, 2, 3, 63, 1e4, None) == INV      # odd d_r
    assert r(None, A, 0, A, 4, 1, 2, 3, 64, 1e4, None) == INV
    assert r(A, A + 4, 0, A, 4, 1, 2, 3, 64, 1e4, None) == INV  # misaligned
    assert r(A, A, 0, A, -1, 1, 2, 3, 64, 1e4, None) == INV


def test_argmax_rows_rejects_before_launch():
    f = tv.load().tv_argmax_rows
    assert f(A, 0, 0, 10, A, None) == OK                   # no rows: nothing to do
    assert f(None, 0, 3, 10, A, None) == INV
    assert f(A, 0, 3, 10, None, None) == INV
    assert f(A, 0, 3, 0, A, None) == INV                   # empty vocabulary
    assert f(A, 0, -1, 10, A, None) == INV
    assert f(A, 5, 3, 10, A, None) == INV                  # dtype
    assert f(A + 2, 0, 3, 10, A, None) == INV              # f32 logits not 4-byte aligned
    assert f(A + 1, 1, 3, 10, A, None) == INV              # bf16 logits not 2-byte aligned
    assert f(A, 0, 3, 10, A + 2, None) == INV
    assert f(A, 0, 2**31, 10, A, None) == UNS


def test_tree_accept_rejects_before_launch():
    f = tv.load().tv_tree_accept
    assert f(None, A, A, 1, 3, A, A, A, None) == INV
    assert f(A, A, A, 0, 3, A, A, A, None) == INV
    assert f(A, A, A, 1, 0, A, A, A, None) == INV
    assert f(A, A, A, 1, 257, A, A, A, None) == UNS
    assert f(A, A, A + 2, 1, 3, A, A, A, None) == INV
    assert f(A, A, A, 1, 3, A, None, A, None) == INV


def test_kv_compact_rejects_before_launch():
    f = tv.load().tv_kv_compact
    assert f(None, A, 1, A, A, 4, 1, 7, 3, 512, 64, None) == INV
    assert f(A, A, 1, A, A, 5, 1, 7, 3, 512, 64, None) == INV          # prefix + q_len > kv_len
    assert f(A, A, 1, A, A, 4, 1, 7, 257, 512, 64, None) == UNS
    assert f(A, A, 1, A, A, 4, 1, 7, 3, 12, 64, None) == UNS           # 24-byte rows
    assert f(A + 8, A, 1, A, A, 4, 1, 7, 3, 512, 64, None) == INV      # c_kv not 16-byte aligned
    assert f(A, A, 9, A, A, 4, 1, 7, 3, 512, 64, None) == INV          # dtype


def test_tree_build_rejects_before_launch():
    lib = tv.load()
    f = lib.tv_tree_build
    args = lambda B=2, D=4, K=8, budget=32, lp=A, out=A: (lp, A, A, B, D, K, budget, out, A, A, A, A, None)
    assert f(*args(K=0)) == INV
    assert f(*args(K=65)) == UNS
    assert f(*args(D=0)) == INV
    assert f(*args(B=0)) == INV
    assert f(*args(budget=-1)) == INV
    assert f(*args(budget=256)) == UNS
    assert f(*args(D=200, K=64, budget=200)) == UNS   # 12800 ranked candidates
    assert f(*args(D=128, K=65, budget=200)) == UNS
    assert f(*args(lp=None)) == INV
    assert f(*args(lp=A + 2)) == INV
    assert f(*args(out=None)) == INV


def test_verify_attn_ragged_rejects_before_launch():
    lib = tv.load()
    ws_size = lib.tv_verify_attn_ragged_workspace_size
    assert ws_size(3, 8, 33, 9000, 512, 64, 1) > 0
    assert ws_size(3, 8, 33, 20, 512, 64, 1) == 0        # stride below max_q_len
    assert ws_size(3, 8, 257, 9000, 512, 64, 1) == 0     # tree too large
    need = ws_size(3, 8, 33, 9000, 512, 64, 1)
    f = lib.tv_verify_attn_ragged

    def call(**kw):
        a = dict(q=A, p=A, N=40, B=3, H=8, mq=33, S=9000, d_c=512, d_r=64, dt=1, ws=A, ws_n=need)
        a.update(kw)
        return f(a["q"], A, A, A, A, a["p"], A, a["N"], a["B"], a["H"], a["mq"], a["S"], a["d_c"], a["d_r"],
                 a["dt"], 0.04, A, None, a["ws"], a["ws_n"], None)

    assert call(S=20) == INV
    assert call(mq=257) == UNS
    assert call(B=0) == INV
    assert call(q=None) == INV
    assert call(p=None) == INV
    assert call(p=A + 2) == INV
    assert call(ws=None) == INV
    assert call(ws_n=need - 1) == INV
    assert call(ws=A + 8) == INV
    assert call(d_c=100) == UNS
    assert call(N=-1) == INV                              # negative node count
    assert call(N=2**28) == UNS                           # N * H rows past int32


def test_verify_attn_noalloc_rejects_before_launch():
    """The no-allocation entry point checks its arguments like tv_verify_attn,
    and a shape whose split-kv scratch exceeds the static array is refused
    before any device call."""
    lib = tv.load()
    f = lib.tv_verify_attn_noalloc

    def call(prefix=4, B=1, H=2, q=3, d_c=64, d_r=32, dt=0, out=A, q_lat=A):
        return f(q_lat, A, A, A, A, prefix, B, H, q, d_c, d_r, dt, 0.1, out, None, None)

    assert call(out=None) == INV
    assert call(q_lat=A + 8) == INV
    assert call(B=0) == INV
    assert call(q=257) == UNS
    assert call(d_c=100) == UNS
    # four long trees: every row block cut into many kv pieces, ~268 MB of partials
    need = tv.workspace_size(4, 64, 33, 200000, 512, 64, tv.TV_BF16)
    assert need > tv.TV_NOALLOC_SCRATCH_BYTES
    assert call(prefix=200000, B=4, H=64, q=33, d_c=512, d_r=64, dt=1) == UNS
    # the serving batch fits the array
    assert 0 < tv.workspace_size(32, 64, 33, 8192, 512, 64, tv.TV_BF16) <= tv.TV_NOALLOC_SCRATCH_BYTES


def test_verify_attn_ex_flags():
    """tv_verify_attn_ex: flags 0 is tv_verify_attn; TV_ATTN_BF16_QUERIES
    selects the one-term query kernel (its own workspace size) and
    TV_ATTN_F32_WIDE the fp32 kernel's 64-row form (its own workspace size for
    a small batch); unknown bits are refused before launch."""
    lib = tv.load()
    f = lib.tv_verify_attn_ex
    assert (tv.TV_ATTN_BF16_QUERIES, tv.TV_ATTN_F32_WIDE) == (1, 2)
    assert f(A, A, A, A, A, 4, 1, 2, 3, 64, 32, 0, 0.1, 4, A, None, None, 0, None) == INV     # unknown flag
    assert f(A, A, A, A, A, 4, 1, 2, 3, 64, 32, 0, 0.1, 1 << 31, A, None, None, 0, None) == INV
    assert f(None, A, A, A, A, 4, 1, 2, 3, 64, 32, 0, 0.1, 1, A, None, None, 0, None) == INV
    assert f(A, A, A, A, A, 4, 1, 2, 257, 64, 32, 0, 0.1, 1, A, None, None, 0, None) == UNS
    ws = lib.tv_verify_attn_ex_workspace_size
    assert ws(32, 64, 33, 8192, 512, 64, 1, 4) == 0                   # unknown flag
    # serving batch: 64-row blocks with two-term queries, 128-row blocks with one
    two, one = ws(32, 64, 33, 8192, 512, 64, 1, 0), ws(32, 64, 33, 8192, 512, 64, 1, 1)
    assert two == tv.workspace_size(32, 64, 33, 8192, 512, 64, tv.TV_BF16) and 0 < two < one
    # the bf16-queries flag changes nothing for the fp32 cache, the wide flag
    # nothing for the bf16 cache
    assert ws(2, 64, 9, 5000, 512, 64, 0, 1) == ws(2, 64, 9, 5000, 512, 64, 0, 0)
    assert ws(32, 64, 33, 8192, 512, 64, 1, 2) == two and ws(32, 64, 33, 8192, 512, 64, 1, 3) == one
    # a small fp32 batch: 32-row blocks by default (two splits' partials per
    # 64 rows of the wide form's one), the wide form on request
    narrow, wide = ws(2, 64, 9, 5000, 512, 64, 0, 0), ws(2, 64, 9, 5000, 512, 64, 0, 2)
    assert narrow > 0 and wide > 0 and narrow != wide
    # a batch of more than 128 64-row blocks takes the wide form either way
    assert ws(3, 64, 44, 5000, 512, 64, 0, 0) == ws(3, 64, 44, 5000, 512, 64, 0, 2)
