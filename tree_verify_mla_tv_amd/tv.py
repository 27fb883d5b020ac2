"""Thin Python binding of libtv.so (ctypes): argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI of include/tv.h;
PyTorch only provides device memory and the current stream.  If libtv.so is
missing the calls raise: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtv.so")

TV_OK, TV_ERR_INVALID, TV_ERR_UNSUPPORTED, TV_ERR_LAUNCH = 0, 1, 2, 3
TV_ATTN_BF16_QUERIES = 1
TV_ATTN_F32_WIDE = 2
TV_F32, TV_BF16 = 0, 1
TV_MAX_Q_LEN = 256
TV_MAX_BUILD_BUDGET = TV_MAX_Q_LEN - 1
TV_MAX_BUILD_CANDIDATES = 8192
TV_NOALLOC_SCRATCH_BYTES = 80 << 20

_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_f64 = ctypes.c_double
_sz = ctypes.c_size_t

SIGNATURES = {
    "tv_status_str": (ctypes.c_char_p, [_i32]),
    "tv_tree_positions": (_i32, [_p, _i32, _i32, _i32, _p, _p]),
    "tv_rope_neox": (_i32, [_p, _i32, _p, _i64, _i32, _i32, _i64, _f64, _p]),
    "tv_rope_neox_strided": (_i32, [_p, _i32, _p, _i32, _i32, _i32, _i32, _i64, _i64, _i64, _f64, _p]),
    "tv_verify_attn": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p,
                              _sz, _p]),
    "tv_verify_attn_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "tv_verify_attn_ex": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                 ctypes.c_uint32, _p, _p, _p, _sz, _p]),
    "tv_verify_attn_ex_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_uint32]),
    "tv_verify_attn_noalloc": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p,
                                      _p]),
    "tv_tree_rope": (_i32, [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _f64, _p]),
    "tv_verify_step": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f64, _f32, _p, _p,
                              _p, _sz, _p]),
    "tv_argmax_rows": (_i32, [_p, _i32, _i64, _i32, _p, _p]),
    "tv_tree_accept": (_i32, [_p, _p, _p, _i32, _i32, _p, _p, _p, _p]),
    "tv_kv_compact": (_i32, [_p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p]),
    "tv_tree_build": (_i32, [_p, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p]),
    "tv_verify_attn_ragged": (_i32, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _f32, _p, _p, _p, _sz, _p]),
    "tv_verify_attn_ragged_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "tv_verify_step_ragged": (_i32, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _f64, _f32, _p, _p, _p, _sz, _p]),
}


class TVError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {status_str(code)}")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m tree_verify_mla_tv_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_str(code: int) -> str:
    return load().tv_status_str(code).decode()


def _check(fn: str, code: int):
    if code != TV_OK:
        raise TVError(fn, code)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TV_F32
    if t.dtype == torch.bfloat16:
        return TV_BF16
    raise TypeError(f"cache dtype must be float32 or bfloat16, got {t.dtype}")


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _cuda_contig(name: str, t: torch.Tensor):
    _need(t.is_cuda, f"{name} must be a CUDA (HIP) tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def tree_positions(parent: torch.Tensor, prefix_len: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """pos[b, i] = prefix_len + depth(i) for parent arrays [B, q_len] (int32)."""
    _cuda_contig("parent", parent)
    _need(parent.dtype == torch.int32 and parent.dim() == 2, "parent must be int32 [B, q_len]")
    B, q = parent.shape
    if out is None:
        out = torch.empty_like(parent)
    _check("tv_tree_positions", load().tv_tree_positions(_ptr(parent), B, q, prefix_len, _ptr(out), _stream()))
    return out


def rope_neox(x: torch.Tensor, pos: torch.Tensor | None = None, theta: float = 10000.0) -> torch.Tensor:
    """In-place NeoX RoPE (float64 angles) of x [n_tok, (n_head,) d_r]: tv_rope_neox.

    The head and feature axes must be dense; the token axis may be strided.
    pos: int32 [n_tok] contiguous, or None for position = token index.
    """
    _need(x.is_cuda, "x must be a CUDA tensor")
    if x.dim() == 2:
        n_tok, d_r = x.shape
        n_head = 1
    else:
        _need(x.dim() == 3, "x must be [n_tok, n_head, d_r] or [n_tok, d_r]")
        n_tok, n_head, d_r = x.shape
        _need(n_head == 1 or x.stride(1) == d_r, "heads of x must be dense rows")
    _need(x.stride(-1) == 1, "the feature axis of x must be contiguous")
    dt = _kv_dtype(x)
    if pos is not None:
        _need(pos.is_cuda and pos.dtype == torch.int32 and pos.shape == (n_tok,) and pos.is_contiguous(),
              "pos must be contiguous CUDA int32 [n_tok]")
    _check("tv_rope_neox", load().tv_rope_neox(_ptr(x), dt, _ptr(pos), n_tok, n_head, d_r, x.stride(0),
                                               float(theta), _stream()))
    return x


def rope_neox_strided(x: torch.Tensor, pos: torch.Tensor | None = None, theta: float = 10000.0) -> torch.Tensor:
    """In-place NeoX RoPE (float64 angles) of x [n_seq, n_tok, (n_head,) d_r]:
    tv_rope_neox_strided.

    The head and feature axes must be dense; the sequence and token axes may be
    strided (e.g. a slice of a kv cache).  pos: int32 [n_seq, n_tok] (row stride
    free), or None for position = token index.
    """
    _need(x.is_cuda, "x must be a CUDA tensor")
    if x.dim() == 3:
        n_seq, n_tok, d_r = x.shape
        n_head = 1
    else:
        _need(x.dim() == 4, "x must be [n_seq, n_tok, n_head, d_r] or [n_seq, n_tok, d_r]")
        n_seq, n_tok, n_head, d_r = x.shape
        _need(n_head == 1 or x.stride(2) == d_r, "heads of x must be dense rows")
    _need(x.stride(-1) == 1, "the feature axis of x must be contiguous")
    dt = _kv_dtype(x)
    pos_stride = 0
    if pos is not None:
        _need(pos.is_cuda and pos.dtype == torch.int32 and pos.shape == (n_seq, n_tok) and pos.stride(1) == 1,
              "pos must be CUDA int32 [n_seq, n_tok] with unit token stride")
        pos_stride = pos.stride(0)
    _check("tv_rope_neox_strided", load().tv_rope_neox_strided(_ptr(x), dt, _ptr(pos), n_seq, n_tok, n_head, d_r,
                                                               x.stride(0), x.stride(1), pos_stride, float(theta),
                                                               _stream()))
    return x


def workspace_size(B: int, H: int, q_len: int, prefix_len: int, d_c: int, d_r: int, kv_dtype: int,
                   flags: int = 0) -> int:
    if flags:
        return int(load().tv_verify_attn_ex_workspace_size(B, H, q_len, prefix_len, d_c, d_r, kv_dtype, flags))
    return int(load().tv_verify_attn_workspace_size(B, H, q_len, prefix_len, d_c, d_r, kv_dtype))


def _attn_shapes(q_lat, q_rope, c_kv, k_rope, parent, prefix_len):
    for n, t in (("q_lat", q_lat), ("q_rope", q_rope), ("c_kv", c_kv), ("k_rope", k_rope), ("parent", parent)):
        _cuda_contig(n, t)
    _need(q_lat.dtype == torch.float32 and q_rope.dtype == torch.float32, "q_lat and q_rope must be float32")
    _need(parent.dtype == torch.int32, "parent must be int32")
    _need(c_kv.dtype == k_rope.dtype, "c_kv and k_rope must share a dtype")
    B, q, H, d_c = q_lat.shape
    d_r = q_rope.shape[-1]
    kv = prefix_len + q
    _need(q_rope.shape == (B, q, H, d_r), f"q_rope must be {(B, q, H, d_r)}")
    _need(c_kv.shape == (B, kv, d_c), f"c_kv must be {(B, kv, d_c)}")
    _need(k_rope.shape == (B, kv, d_r), f"k_rope must be {(B, kv, d_r)}")
    _need(parent.shape == (B, q), f"parent must be {(B, q)}")
    return B, q, H, d_c, d_r


def _outputs(q_lat, out, lse, return_lse, workspace, ws_bytes):
    B, q, H, d_c = q_lat.shape
    if out is None:
        out = torch.empty_like(q_lat)
    else:
        _cuda_contig("out", out)
        _need(out.shape == q_lat.shape and out.dtype == torch.float32, "out must be float32 like q_lat")
    if lse is None and return_lse:
        lse = torch.empty((B, q, H), dtype=torch.float32, device=q_lat.device)
    if lse is not None:
        _cuda_contig("lse", lse)
        _need(lse.shape == (B, q, H) and lse.dtype == torch.float32, "lse must be float32 [B, q_len, H]")
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q_lat.device)
    if workspace is not None:
        _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous CUDA tensor")
    return out, lse, workspace


def verify_attn(q_lat, q_rope, c_kv, k_rope, parent, prefix_len: int, sm_scale: float | None = None, out=None,
                lse=None, return_lse: bool = False, workspace=None):
    """Tree-verify MLA-absorb attention (rope slices already rotated): tv_verify_attn.

    Returns out [B, q_len, H, d_c] float32 (and lse [B, q_len, H] if asked or given).
    sm_scale defaults to 1/sqrt(d_c + d_r), rounded to fp32.
    """
    return verify_attn_ex(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, sm_scale, 0, out, lse, return_lse,
                          workspace)


def verify_attn_ex(q_lat, q_rope, c_kv, k_rope, parent, prefix_len: int, sm_scale: float | None = None,
                   flags: int = 0, out=None, lse=None, return_lse: bool = False, workspace=None):
    """verify_attn with option flags (tv_verify_attn_ex; flags 0 calls
    tv_verify_attn).  TV_ATTN_BF16_QUERIES rounds the scaled queries to one
    bf16 term on the bf16-cache matrix-core path; TV_ATTN_F32_WIDE keeps an
    fp32-cache batch at (512, 64) on the 64-row workgroups at every size."""
    B, q, H, d_c, d_r = _attn_shapes(q_lat, q_rope, c_kv, k_rope, parent, prefix_len)
    dt = _kv_dtype(c_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_c + d_r)
    ws_bytes = workspace_size(B, H, q, prefix_len, d_c, d_r, dt, flags)
    out, lse_t, workspace = _outputs(q_lat, out, lse, return_lse, workspace, ws_bytes)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(q_lat), _ptr(q_rope), _ptr(c_kv), _ptr(k_rope), _ptr(parent), prefix_len, B, H, q, d_c, d_r, dt,
            float(sm_scale))
    tail = (_ptr(out), _ptr(lse_t), _ptr(workspace), ws_n, _stream())
    if flags:
        _check("tv_verify_attn_ex", load().tv_verify_attn_ex(*head, flags, *tail))
    else:
        _check("tv_verify_attn", load().tv_verify_attn(*head, *tail))
    return (out, lse_t) if (return_lse or lse is not None) else out


def verify_attn_noalloc(q_lat, q_rope, c_kv, k_rope, parent, prefix_len: int, sm_scale: float | None = None,
                        out=None, lse=None, return_lse: bool = False):
    """verify_attn through tv_verify_attn_noalloc: the split-kv scratch is the
    library's static device array (no workspace).  out / lse must be given for
    a call that may not allocate; when they are None they are allocated here,
    before the library call."""
    B, q, H, d_c, d_r = _attn_shapes(q_lat, q_rope, c_kv, k_rope, parent, prefix_len)
    dt = _kv_dtype(c_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_c + d_r)
    out, lse_t, _ = _outputs(q_lat, out, lse, return_lse, None, 0)
    _check("tv_verify_attn_noalloc", load().tv_verify_attn_noalloc(
        _ptr(q_lat), _ptr(q_rope), _ptr(c_kv), _ptr(k_rope), _ptr(parent), prefix_len, B, H, q, d_c, d_r, dt,
        float(sm_scale), _ptr(out), _ptr(lse_t), _stream()))
    return (out, lse_t) if (return_lse or lse is not None) else out


def verify_attn_ragged(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, q_len, max_q_len: int,
                       sm_scale: float | None = None, out=None, lse=None, return_lse: bool = False, workspace=None):
    """Tree-verify attention over requests of different lengths (rope slices
    already rotated).  Nodes packed request after request: q_lat [N, H, d_c],
    q_rope [N, H, d_r], parent [N] int32 (local node indices); cache c_kv
    [B, kv_stride, d_c], k_rope [B, kv_stride, d_r]; prefix_len and q_len: int32
    [B] device tensors (q_len[b] <= max_q_len, prefix_len[b] + q_len[b] <=
    kv_stride).  N (the rows of q_lat) bounds the packed nodes: if the lengths
    sum to more, the request crossing N keeps its nodes below N and later
    requests get none.  Returns out [N, H, d_c] (and lse [N, H])."""
    return _ragged("tv_verify_attn_ragged", q_lat, q_rope, c_kv, k_rope, parent, prefix_len, q_len, max_q_len,
                   sm_scale, out, lse, return_lse, workspace, None)


def _ragged(fn, q_lat, q_rope, c_kv, k_rope, parent, prefix_len, q_len, max_q_len, sm_scale, out, lse, return_lse,
            workspace, theta):
    for n, t in (("q_lat", q_lat), ("q_rope", q_rope), ("c_kv", c_kv), ("k_rope", k_rope), ("parent", parent),
                 ("prefix_len", prefix_len), ("q_len", q_len)):
        _cuda_contig(n, t)
    _need(q_lat.dtype == torch.float32 and q_lat.dim() == 3, "q_lat must be float32 [N, H, d_c]")
    N, H, d_c = q_lat.shape
    _need(q_rope.dtype == torch.float32 and q_rope.dim() == 3 and q_rope.shape[:2] == (N, H),
          "q_rope must be float32 [N, H, d_r]")
    d_r = q_rope.shape[2]
    _need(c_kv.dim() == 3 and c_kv.shape[2] == d_c, "c_kv must be [B, kv_stride, d_c]")
    B, S = c_kv.shape[:2]
    _need(k_rope.shape == (B, S, d_r) and k_rope.dtype == c_kv.dtype, "k_rope must be [B, kv_stride, d_r] like c_kv")
    _need(parent.dtype == torch.int32 and parent.shape == (N,), "parent must be int32 [N]")
    _need(prefix_len.dtype == torch.int32 and prefix_len.shape == (B,), "prefix_len must be int32 [B]")
    _need(q_len.dtype == torch.int32 and q_len.shape == (B,), "q_len must be int32 [B]")
    dt = _kv_dtype(c_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_c + d_r)
    ws_bytes = load().tv_verify_attn_ragged_workspace_size(B, H, max_q_len, S, d_c, d_r, dt)
    _need(ws_bytes > 0, "unsupported shape for the ragged attention")
    if out is None:
        out = torch.empty_like(q_lat)
    _cuda_contig("out", out)
    _need(out.dtype == torch.float32 and out.shape == (N, H, d_c), "out must be float32 [N, H, d_c]")
    if lse is None and return_lse:
        lse = torch.empty(N, H, dtype=torch.float32, device=q_lat.device)
    if lse is not None:
        _cuda_contig("lse", lse)
        _need(lse.dtype == torch.float32 and lse.shape == (N, H), "lse must be float32 [N, H]")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q_lat.device)
    ws_n = workspace.numel() * workspace.element_size()
    head = (_ptr(q_lat), _ptr(q_rope), _ptr(c_kv), _ptr(k_rope), _ptr(parent), _ptr(prefix_len), _ptr(q_len), N, B,
            H, max_q_len, S, d_c, d_r, dt)
    tail = (float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_n, _stream())
    args = head + tail if theta is None else head + (float(theta),) + tail
    _check(fn, getattr(load(), fn)(*args))
    return (out, lse) if (return_lse or lse is not None) else out


def verify_step_ragged(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, q_len, max_q_len: int,
                       theta: float = 10000.0, sm_scale: float | None = None, out=None, lse=None,
                       return_lse: bool = False, workspace=None):
    """The whole step for a ragged batch: rotate each request's q_rope rows and
    tree key rows in place at prefix_len[b] + depth, then the ragged attention
    (arguments as for verify_attn_ragged)."""
    return _ragged("tv_verify_step_ragged", q_lat, q_rope, c_kv, k_rope, parent, prefix_len, q_len, max_q_len,
                   sm_scale, out, lse, return_lse, workspace, theta)


def tree_rope(q_rope, k_rope, parent, prefix_len: int, theta: float = 10000.0):
    """Rotate q_rope [B,q,H,d_r] and the tree's key rows k_rope[:, prefix_len:, :]
    in place at prefix_len + depth(node) (one fused launch)."""
    _cuda_contig("q_rope", q_rope)
    _cuda_contig("k_rope", k_rope)
    _cuda_contig("parent", parent)
    _need(q_rope.dtype == torch.float32 and q_rope.dim() == 4, "q_rope must be float32 [B, q_len, H, d_r]")
    _need(parent.dtype == torch.int32, "parent must be int32")
    B, q, H, d_r = q_rope.shape
    _need(k_rope.shape == (B, prefix_len + q, d_r), f"k_rope must be {(B, prefix_len + q, d_r)}")
    _need(parent.shape == (B, q), f"parent must be {(B, q)}")
    _check("tv_tree_rope", load().tv_tree_rope(_ptr(q_rope), _ptr(k_rope), _kv_dtype(k_rope), _ptr(parent),
                                               prefix_len, B, H, q, d_r, float(theta), _stream()))
    return q_rope, k_rope


def verify_step(q_lat, q_rope, c_kv, k_rope, parent, prefix_len: int, theta: float = 10000.0,
                sm_scale: float | None = None, out=None, lse=None, return_lse: bool = False, workspace=None):
    """The whole step: rotate q_rope and the tree's key rows in place at
    prefix_len + depth, then tree-verify attention.  Prefix key rows are taken
    as already rotated."""
    B, q, H, d_c, d_r = _attn_shapes(q_lat, q_rope, c_kv, k_rope, parent, prefix_len)
    dt = _kv_dtype(c_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_c + d_r)
    ws_bytes = workspace_size(B, H, q, prefix_len, d_c, d_r, dt)
    out, lse_t, workspace = _outputs(q_lat, out, lse, return_lse, workspace, ws_bytes)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tv_verify_step", load().tv_verify_step(
        _ptr(q_lat), _ptr(q_rope), _ptr(c_kv), _ptr(k_rope), _ptr(parent), prefix_len, B, H, q, d_c, d_r, dt,
        float(theta), float(sm_scale), _ptr(out), _ptr(lse_t), _ptr(workspace), ws_n, _stream()))
    return (out, lse_t) if (return_lse or lse is not None) else out


def argmax_rows(logits: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """The target's greedy token per row of logits [..., vocab] (float32 or
    bfloat16): int32 [...], lowest index on ties, a NaN beats every number."""
    _cuda_contig("logits", logits)
    dt = _kv_dtype(logits)
    vocab = logits.shape[-1]
    n_rows = logits.numel() // vocab
    if out is None:
        out = torch.empty(logits.shape[:-1], dtype=torch.int32, device=logits.device)
    _cuda_contig("out", out)
    _need(out.dtype == torch.int32 and out.numel() == n_rows, "out must be int32 with one entry per row")
    _check("tv_argmax_rows", load().tv_argmax_rows(_ptr(logits), dt, n_rows, vocab, _ptr(out), _stream()))
    return out


def tree_accept(parent: torch.Tensor, draft_tok: torch.Tensor, target_tok: torch.Tensor):
    """Greedy acceptance per tree: returns (path [B, q] int32, accept_len [B]
    int32, bonus [B] int32).  All inputs int32 [B, q_len]."""
    for n, t in (("parent", parent), ("draft_tok", draft_tok), ("target_tok", target_tok)):
        _cuda_contig(n, t)
        _need(t.dtype == torch.int32 and t.dim() == 2, f"{n} must be int32 [B, q_len]")
    B, q = parent.shape
    _need(draft_tok.shape == (B, q) and target_tok.shape == (B, q), "inputs must share the shape [B, q_len]")
    path = torch.empty_like(parent)
    accept_len = torch.empty(B, dtype=torch.int32, device=parent.device)
    bonus = torch.empty(B, dtype=torch.int32, device=parent.device)
    _check("tv_tree_accept", load().tv_tree_accept(_ptr(parent), _ptr(draft_tok), _ptr(target_tok), B, q, _ptr(path),
                                                   _ptr(accept_len), _ptr(bonus), _stream()))
    return path, accept_len, bonus


def kv_compact(c_kv: torch.Tensor, k_rope: torch.Tensor, path: torch.Tensor, accept_len: torch.Tensor,
               prefix_len: int):
    """Move the accepted nodes' rows of c_kv [B, kv, d_c] and k_rope [B, kv, d_r]
    to rows prefix_len + 1 .. prefix_len + accept_len, in place."""
    for n, t in (("c_kv", c_kv), ("k_rope", k_rope), ("path", path), ("accept_len", accept_len)):
        _cuda_contig(n, t)
    _need(c_kv.dtype == k_rope.dtype, "c_kv and k_rope must share a dtype")
    _need(path.dtype == torch.int32 and accept_len.dtype == torch.int32, "path and accept_len must be int32")
    B, kv, d_c = c_kv.shape
    _need(k_rope.dim() == 3 and k_rope.shape[:2] == (B, kv), "k_rope must be [B, kv, d_r]")
    _need(path.dim() == 2 and path.shape[0] == B and accept_len.shape == (B,), "path [B, q_len], accept_len [B]")
    q = path.shape[1]
    _check("tv_kv_compact", load().tv_kv_compact(_ptr(c_kv), _ptr(k_rope), _kv_dtype(c_kv), _ptr(path),
                                                 _ptr(accept_len), prefix_len, B, kv, q, d_c, k_rope.shape[2],
                                                 _stream()))
    return c_kv, k_rope


def tree_build(logp: torch.Tensor, cand_tok: torch.Tensor, root_tok: torch.Tensor, budget: int):
    """Best-first draft tree per request from the drafter's proposals: logp
    float32 [B, D, K], cand_tok int32 [B, D, K], root_tok int32 [B].  Returns
    (parent, token, depth, score) each [B, budget + 1] (int32, int32, int32,
    float32) and n_nodes [B] int32."""
    _cuda_contig("logp", logp)
    _cuda_contig("cand_tok", cand_tok)
    _cuda_contig("root_tok", root_tok)
    _need(logp.dtype == torch.float32 and logp.dim() == 3, "logp must be float32 [B, D, K]")
    _need(cand_tok.dtype == torch.int32 and cand_tok.shape == logp.shape, "cand_tok must be int32 like logp")
    B, D, K = logp.shape
    _need(root_tok.dtype == torch.int32 and root_tok.shape == (B,), "root_tok must be int32 [B]")
    dev = logp.device
    q = budget + 1
    parent = torch.empty(B, q, dtype=torch.int32, device=dev)
    token = torch.empty(B, q, dtype=torch.int32, device=dev)
    depth = torch.empty(B, q, dtype=torch.int32, device=dev)
    score = torch.empty(B, q, dtype=torch.float32, device=dev)
    n_nodes = torch.empty(B, dtype=torch.int32, device=dev)
    _check("tv_tree_build", load().tv_tree_build(_ptr(logp), _ptr(cand_tok), _ptr(root_tok), B, D, K, budget,
                                                 _ptr(parent), _ptr(token), _ptr(depth), _ptr(score),
                                                 _ptr(n_nodes), _stream()))
    return parent, token, depth, score, n_nodes
