"""ctypes binding of libattn.so.

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, turned into device pointers and sizes, and handed to the C ABI on the
caller's current stream. Every step of the computation runs in the HIP
kernels; there is no fallback path. If the shared library is missing the
import fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIB_PATH selects another build of the same library (the host-sanitized
# test build of the C ABI layer); by default the in-tree libattn.so.
LIB_PATH = os.environ.get("ATTN_LIB_PATH") or os.path.join(_PKG, "libattn.so")

ATTN_OK, ATTN_E_ARG, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP = range(5)
ATTN_F32, ATTN_BF16 = 0, 1
ATTN_PAGES_TOKEN_MAJOR, ATTN_PAGES_HEAD_MAJOR = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python transformer_attention_split_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float

lib.attn_status_str.restype = ctypes.c_char_p
lib.attn_status_str.argtypes = [_i]
lib.attn_last_error.restype = ctypes.c_char_p
lib.attn_last_error.argtypes = []
lib.attn_abi_version.restype = _i
lib.attn_abi_version.argtypes = []
lib.attn_decode_workspace_bytes.restype = _sz
lib.attn_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
lib.attn_decode.restype = _i
lib.attn_decode.argtypes = [_i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p,
                            _f, _i, _p, _sz, _p]
lib.attn_decode_noalloc.restype = _i
lib.attn_decode_noalloc.argtypes = [_i, _p, _p, _p, _p, _i, _i, _i, _i, _i,
                                    _i, _p, _f, _i, _p]
lib.attn_decode_append.restype = _i
lib.attn_decode_append.argtypes = [_i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i,
                                   _i, _i, _p, _f, _i, _p, _sz, _p]
lib.attn_decode_append_rope.restype = _i
lib.attn_decode_append_rope.argtypes = [_i, _p, _p, _p, _p, _p, _p, _p, _p, _i,
                                        _i, _i, _i, _i, _i, _p, _f, _i, _p,
                                        _sz, _p]
lib.attn_decode_paged.restype = _i
lib.attn_decode_paged.argtypes = [_i, _p, _p, _p, _p, _i, _i, _i, _i, _p, _i,
                                  _i, _i, _i, _i, _p, _f, _i, _p, _sz, _p]
lib.attn_prefill.restype = _i
lib.attn_prefill.argtypes = [_i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                             _f, _p]
lib.attn_prefill_paged.restype = _i
lib.attn_prefill_paged.argtypes = [_i, _p, _p, _p, _p, _i, _i, _i, _i, _p, _i,
                                   _i, _i, _i, _i, _i, _f, _p]
lib.attn_topk.restype = _i
lib.attn_topk.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
lib.attn_topk_causal.restype = _i
lib.attn_topk_causal.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
lib.attn_read_probe.restype = _i
lib.attn_read_probe.argtypes = [_p, _sz, _p, _sz, _i, _p]

EXPORTED = ("attn_status_str", "attn_last_error", "attn_abi_version",
            "attn_decode_workspace_bytes", "attn_decode", "attn_decode_noalloc",
            "attn_decode_append",
            "attn_decode_append_rope",
            "attn_decode_paged", "attn_prefill", "attn_prefill_paged",
            "attn_topk",
            "attn_topk_causal", "attn_read_probe")


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.attn_status_str(status).decode()
        detail = lib.attn_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" — {detail}" if detail else ""))


class AttnArgError(AttnError, ValueError):
    pass


def _check(status: int, where: str) -> None:
    if status == ATTN_OK:
        return
    if status in (ATTN_E_ARG, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE):
        raise AttnArgError(status, where)
    raise AttnError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _resolve_stream(stream) -> torch.cuda.Stream:
    """The stream the kernels are enqueued on, as a torch stream object:
    the current stream for None, the object itself for a torch stream, and
    an ExternalStream around a raw hipStream_t handle (int) or an object with
    a ``cuda_stream`` attribute."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if not h:
        return torch.cuda.default_stream()
    return torch.cuda.ExternalStream(h)


def _handle(s: torch.cuda.Stream) -> Optional[int]:
    return s.cuda_stream or None


def _guard(s: torch.cuda.Stream, *owned: Optional[torch.Tensor]) -> None:
    """Tensors this wrapper allocated (workspace, output, ...) come from the
    caching allocator on the current stream. When the kernels run on another
    stream, record that use: otherwise, once the wrapper drops its reference,
    the allocator may hand the memory to the next allocation on the current
    stream while the kernels still read or write it."""
    if s == torch.cuda.current_stream(s.device):
        return
    for t in owned:
        if t is not None:
            t.record_stream(s)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _need_dense(name: str, t: torch.Tensor, ndim: int) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------
def attn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int,
                                max_length: int, split_rows: int = 0) -> int:
    return int(lib.attn_decode_workspace_bytes(B, Hq, Hkv, D, max_length,
                                               split_rows))


def _decode_args(q, k_cache, v_cache, position_id, seq_lens, scale,
                 split_rows, out, workspace):
    """Shared checks of attn_decode / attn_decode_append; returns the
    marshalled sizes, scale, out and workspace."""
    _need_dense("q", q, 3)
    _need_dense("k_cache", k_cache, 4)
    _need_dense("v_cache", v_cache, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache and v_cache must share one dtype")
    B, Hq, D = q.shape
    Bk, Hkv, max_length, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match "
                         f"q {tuple(q.shape)}")
    if (position_id is None) == (seq_lens is None):
        raise ValueError("pass exactly one of position_id or seq_lens")
    if seq_lens is not None:
        _need_dense("seq_lens", seq_lens, 1)
        if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
            raise ValueError("seq_lens must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    owned = []
    if out is None:
        out = torch.empty_like(q)
        owned.append(out)
    else:
        _need_dense("out", out, 3)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q's shape and dtype")
    need = attn_decode_workspace_bytes(B, Hq, Hkv, D, max_length, split_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8,
                                device=q.device)
        owned.append(workspace)
    return B, Hq, Hkv, D, max_length, float(scale), out, workspace, owned


def attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                *, position_id: Optional[int] = None,
                seq_lens: Optional[torch.Tensor] = None,
                scale: Optional[float] = None, split_rows: int = 0,
                out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Single-token decode. q [B,Hq,D]; caches [B,Hkv,max_length,D];
    exactly one of ``position_id`` (rows [0, position_id]) or ``seq_lens``
    (int32 [B] on the GPU, rows [0, seq_lens[b])). Returns out [B,Hq,D]."""
    B, Hq, Hkv, D, max_length, scale, out, workspace, owned = _decode_args(
        q, k_cache, v_cache, position_id, seq_lens, scale, split_rows, out,
        workspace)
    s = _resolve_stream(stream)
    st = lib.attn_decode(_dtype_code(q), _ptr(q), _ptr(k_cache),
                         _ptr(v_cache), _ptr(out), B, Hq, Hkv, D, max_length,
                         -1 if position_id is None else int(position_id),
                         _ptr(seq_lens), scale, int(split_rows),
                         _ptr(workspace), workspace.numel(), _handle(s))
    _check(st, "attn_decode")
    _guard(s, *owned)
    return out


def attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, out: torch.Tensor, *,
                        position_id: Optional[int] = None,
                        seq_lens: Optional[torch.Tensor] = None,
                        scale: Optional[float] = None, split_rows: int = 0,
                        stream=None) -> torch.Tensor:
    """attn_decode with the split partials in the library's static scratch
    (no workspace): for callers that cannot allocate. ``out`` [B,Hq,D] is
    required. Calls that may overlap on one GPU race on the scratch."""
    if out is None:
        raise ValueError("attn_decode_noalloc needs out")
    B, Hq, Hkv, D, max_length, scale, out, _, _ = _decode_args(
        q, k_cache, v_cache, position_id, seq_lens, scale, split_rows, out,
        torch.empty(0, dtype=torch.uint8))
    s = _resolve_stream(stream)
    st = lib.attn_decode_noalloc(
        _dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), B,
        Hq, Hkv, D, max_length, -1 if position_id is None else int(position_id),
        _ptr(seq_lens), scale, int(split_rows), _handle(s))
    _check(st, "attn_decode_noalloc")
    return out


def attn_decode_append(q: torch.Tensor, k_new: torch.Tensor,
                       v_new: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, *,
                       position_id: Optional[int] = None,
                       seq_lens: Optional[torch.Tensor] = None,
                       scale: Optional[float] = None, split_rows: int = 0,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Fused append + decode: k_new / v_new [B,Hkv,D] are stored at row
    position_id (or seq_lens[b]-1) of the caches, which are updated in place,
    and the result equals attn_decode on the updated caches."""
    B, Hq, Hkv, D, max_length, scale, out, workspace, owned = _decode_args(
        q, k_cache, v_cache, position_id, seq_lens, scale, split_rows, out,
        workspace)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need_dense(name, t, 3)
        if tuple(t.shape) != (B, Hkv, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [{B},{Hkv},{D}] {q.dtype}")
    s = _resolve_stream(stream)
    st = lib.attn_decode_append(
        _dtype_code(q), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(out), B, Hq, Hkv, D, max_length,
        -1 if position_id is None else int(position_id), _ptr(seq_lens),
        scale, int(split_rows), _ptr(workspace), workspace.numel(),
        _handle(s))
    _check(st, "attn_decode_append")
    _guard(s, *owned)
    return out


def attn_decode_append_rope(q: torch.Tensor, k_new: torch.Tensor,
                            v_new: torch.Tensor, cos: torch.Tensor,
                            sin: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, *,
                            position_id: Optional[int] = None,
                            seq_lens: Optional[torch.Tensor] = None,
                            scale: Optional[float] = None, split_rows: int = 0,
                            out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Rotary embedding + append + decode: q and k_new are rotated with the
    fp32 cos / sin rows [B,D] of each sequence's current position
    (rotate-half pairs j, j+D/2), the rotated key and v_new are stored as in
    ``attn_decode_append`` and the rotated query attends."""
    B, Hq, Hkv, D, max_length, scale, out, workspace, owned = _decode_args(
        q, k_cache, v_cache, position_id, seq_lens, scale, split_rows, out,
        workspace)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need_dense(name, t, 3)
        if tuple(t.shape) != (B, Hkv, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [{B},{Hkv},{D}] {q.dtype}")
    for name, t in (("cos", cos), ("sin", sin)):
        _need_dense(name, t, 2)
        if tuple(t.shape) != (B, D) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [{B},{D}]")
    s = _resolve_stream(stream)
    st = lib.attn_decode_append_rope(
        _dtype_code(q), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cos),
        _ptr(sin), _ptr(k_cache), _ptr(v_cache), _ptr(out), B, Hq, Hkv, D,
        max_length, -1 if position_id is None else int(position_id),
        _ptr(seq_lens), scale, int(split_rows), _ptr(workspace),
        workspace.numel(), _handle(s))
    _check(st, "attn_decode_append_rope")
    _guard(s, *owned)
    return out


def attn_decode_paged(q: torch.Tensor, k_pages: torch.Tensor,
                      v_pages: torch.Tensor, block_table: torch.Tensor, *,
                      layout: str = "token",
                      position_id: Optional[int] = None,
                      seq_lens: Optional[torch.Tensor] = None,
                      scale: Optional[float] = None, split_rows: int = 0,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Decode over a paged cache. q [B,Hq,D] bf16; pages
    [num_pages,page_size,Hkv,D] (layout="token") or [num_pages,Hkv,page_size,D]
    (layout="head"); block_table int32 [B,max_blocks] on the GPU; exactly one
    of position_id or seq_lens. Returns out [B,Hq,D]."""
    _need_dense("q", q, 3)
    _need_dense("k_pages", k_pages, 4)
    _need_dense("v_pages", v_pages, 4)
    _need_dense("block_table", block_table, 2)
    if k_pages.shape != v_pages.shape:
        raise ValueError("k_pages and v_pages shapes differ")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise ValueError("q, k_pages and v_pages must share one dtype")
    if block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32")
    B, Hq, D = q.shape
    if layout == "token":
        num_pages, page_size, Hkv, Dk = k_pages.shape
        code = ATTN_PAGES_TOKEN_MAJOR
    elif layout == "head":
        num_pages, Hkv, page_size, Dk = k_pages.shape
        code = ATTN_PAGES_HEAD_MAJOR
    else:
        raise ValueError("layout must be 'token' or 'head'")
    if Dk != D or block_table.shape[0] != B:
        raise ValueError("page, block-table and query shapes do not match")
    max_blocks = block_table.shape[1]
    if (position_id is None) == (seq_lens is None):
        raise ValueError("pass exactly one of position_id or seq_lens")
    if seq_lens is not None:
        _need_dense("seq_lens", seq_lens, 1)
        if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
            raise ValueError("seq_lens must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    owned = []
    if out is None:
        out = torch.empty_like(q)
        owned.append(out)
    else:
        _need_dense("out", out, 3)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q's shape and dtype")
    need = attn_decode_workspace_bytes(B, Hq, Hkv, D, max_blocks * page_size,
                                       split_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8,
                                device=q.device)
        owned.append(workspace)
    s = _resolve_stream(stream)
    st = lib.attn_decode_paged(
        _dtype_code(q), _ptr(q), _ptr(k_pages), _ptr(v_pages),
        _ptr(block_table), max_blocks, page_size, num_pages, code, _ptr(out),
        B, Hq,
        Hkv, D, -1 if position_id is None else int(position_id),
        _ptr(seq_lens), float(scale), int(split_rows), _ptr(workspace),
        workspace.numel(), _handle(s))
    _check(st, "attn_decode_paged")
    _guard(s, *owned)
    return out


# ----------------------------------------------------------------------------
# Prefill
# ----------------------------------------------------------------------------
def attn_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 *, prefix_len: int, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """Causal prefill. q [B,Hq,Lq,D] bf16; caches [B,Hkv,max_length,D] with
    the new tokens' K/V at rows [prefix_len, prefix_len+Lq). Returns
    out [B,Hq,Lq,D]."""
    _need_dense("q", q, 4)
    _need_dense("k_cache", k_cache, 4)
    _need_dense("v_cache", v_cache, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache and v_cache must share one dtype")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, max_length, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError("cache shape does not match q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    owned = None
    if out is None:
        out = owned = torch.empty_like(q)
    else:
        _need_dense("out", out, 4)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q's shape and dtype")
    s = _resolve_stream(stream)
    st = lib.attn_prefill(_dtype_code(q), _ptr(q), _ptr(k_cache),
                          _ptr(v_cache), _ptr(out), B, Hq, Hkv, D, max_length,
                          Lq, int(prefix_len), float(scale), _handle(s))
    _check(st, "attn_prefill")
    _guard(s, owned)
    return out


def attn_prefill_paged(q: torch.Tensor, k_pages: torch.Tensor,
                       v_pages: torch.Tensor, block_table: torch.Tensor, *,
                       prefix_len: int, layout: str = "token",
                       scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Causal prefill over a paged cache. q [B,Hq,Lq,D] bf16; pages
    [num_pages,page_size,Hkv,D] (layout="token") or [num_pages,Hkv,page_size,D]
    (layout="head"); block_table int32 [B,max_blocks] on the GPU. Returns out
    [B,Hq,Lq,D]."""
    _need_dense("q", q, 4)
    _need_dense("k_pages", k_pages, 4)
    _need_dense("v_pages", v_pages, 4)
    _need_dense("block_table", block_table, 2)
    if k_pages.shape != v_pages.shape:
        raise ValueError("k_pages and v_pages shapes differ")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise ValueError("q, k_pages and v_pages must share one dtype")
    if block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32")
    B, Hq, Lq, D = q.shape
    if layout == "token":
        num_pages, page_size, Hkv, Dk = k_pages.shape
        code = ATTN_PAGES_TOKEN_MAJOR
    elif layout == "head":
        num_pages, Hkv, page_size, Dk = k_pages.shape
        code = ATTN_PAGES_HEAD_MAJOR
    else:
        raise ValueError("layout must be 'token' or 'head'")
    if Dk != D or block_table.shape[0] != B:
        raise ValueError("page, block-table and query shapes do not match")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    owned = None
    if out is None:
        out = owned = torch.empty_like(q)
    else:
        _need_dense("out", out, 4)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q's shape and dtype")
    s = _resolve_stream(stream)
    st = lib.attn_prefill_paged(
        _dtype_code(q), _ptr(q), _ptr(k_pages), _ptr(v_pages),
        _ptr(block_table), block_table.shape[1], page_size, num_pages, code,
        _ptr(out), B, Hq, Hkv, D, Lq, int(prefix_len), float(scale),
        _handle(s))
    _check(st, "attn_prefill_paged")
    _guard(s, owned)
    return out


# ----------------------------------------------------------------------------
# Top-k
# ----------------------------------------------------------------------------
def _topk_call(fn: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               topk: int, out: Optional[torch.Tensor],
               idx_out: Optional[torch.Tensor], stream) -> torch.Tensor:
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_dense(name, t, 4)
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must share one shape")
    b, h, n, d = q.shape
    owned = None
    if out is None:
        out = owned = torch.empty_like(q)
    else:
        _need_dense("out", out, 4)
        if out.shape != q.shape or out.dtype != torch.float32:
            raise ValueError("out must be float32 of q's shape")
    if idx_out is not None:
        _need_dense("idx_out", idx_out, 4)
        if idx_out.dtype != torch.int32 or \
                tuple(idx_out.shape) != (b, h, n, topk):
            raise ValueError("idx_out must be int32 [b,h,n,topk]")
    s = _resolve_stream(stream)
    st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(idx_out),
                          b, h, n, d, int(topk), _handle(s))
    _check(st, fn)
    _guard(s, owned)
    return out


def attn_topk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topk: int,
              *, out: Optional[torch.Tensor] = None,
              idx_out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """Top-k sparse attention. q, k, v float32 [b,h,n,d]. Returns out
    [b,h,n,d]; if ``idx_out`` (int32 [b,h,n,topk]) is given it receives the
    selected indices of each row in ascending order."""
    return _topk_call("attn_topk", q, k, v, topk, out, idx_out, stream)


def attn_topk_causal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     topk: int, *, out: Optional[torch.Tensor] = None,
                     idx_out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Decoder-causal top-k sparse attention: row i chooses among keys
    j <= i, keeping every one when i+1 <= topk, else its topk//2 most recent
    plus the best-scoring older ones. Arguments as ``attn_topk``; rows that
    keep fewer than ``topk`` keys pad ``idx_out`` with -1."""
    return _topk_call("attn_topk_causal", q, k, v, topk, out, idx_out, stream)


# ----------------------------------------------------------------------------
# Streaming-read probe (measurement aid)
# ----------------------------------------------------------------------------
def attn_read_probe(src: torch.Tensor, workgroups: int = 4096, *,
                    sink: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Read every byte of the contiguous device tensor ``src`` once (its
    size a multiple of 16 bytes). Returns ``sink``, int32 [workgroups, 4]:
    row w is the XOR of the 16-byte words workgroup w read."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    owned = None
    if sink is None:
        sink = owned = torch.empty((workgroups, 4), dtype=torch.int32,
                                   device=src.device)
    elif not sink.is_contiguous() or sink.dtype != torch.int32 or \
            sink.numel() < 4 * workgroups:
        raise ValueError("sink must be contiguous int32 with >= 4*workgroups "
                         "elements")
    s = _resolve_stream(stream)
    st = lib.attn_read_probe(_ptr(src), nbytes, _ptr(sink),
                             sink.numel() * 4, int(workgroups), _handle(s))
    _check(st, "attn_read_probe")
    _guard(s, owned)
    return sink
