"""Python binding of libpaged_attn.so (the MI355X paged KV-cache attention library).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI declared in ``include/paged_attn.h``.  PyTorch
provides device memory (outputs, workspace) and the current stream.  There is
no fallback: if the shared library is missing and cannot be built, or a call
fails, an exception is raised.

Functions keep the C names: ``paged_attn_fwd``, ``paged_kv_append``,
``paged_attn_workspace_size``, ``paged_attn_splits_for``,
``paged_attn_num_splits``, ``paged_attn_status_string``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

from . import _build

__all__ = [
    "PagedAttnError", "paged_attn_fwd", "paged_attn_fwd_noalloc", "paged_kv_append", "paged_attn_workspace_size",
    "paged_attn_splits_for", "paged_attn_num_splits", "paged_attn_status_string", "library_path",
    "EXPORTED_SYMBOLS",
]

EXPORTED_SYMBOLS = ("paged_attn_fwd", "paged_attn_fwd_noalloc", "paged_kv_append",
                    "paged_attn_workspace_size", "paged_attn_splits_for", "paged_attn_num_splits",
                    "paged_attn_status_string")
PA_ERR_SCRATCH = 9
NOALLOC_SCRATCH_BYTES = 64 << 20   # the library's static scratch array per device

PA_F16, PA_BF16 = 0, 1
_DTYPE_CODE = {torch.float16: PA_F16, torch.bfloat16: PA_BF16}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({paged_attn_status_string(status)})")


class _Args(ctypes.Structure):
    """Mirror of ``pa_fwd_args``."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("total_q", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32), ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("contig_alloc", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("reserved0", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("cache_seqlens", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("softmax_lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("rotary_cos", ctypes.c_void_p), ("rotary_sin", ctypes.c_void_p),
        ("rotary_dim", ctypes.c_int32), ("rotary_interleaved", ctypes.c_int32),
        ("rotary_rows", ctypes.c_int32), ("reserved1", ctypes.c_int32),
        ("q_row_stride", ctypes.c_int64), ("k_new_row_stride", ctypes.c_int64),
        ("v_new_row_stride", ctypes.c_int64), ("aux_stream", ctypes.c_void_p),
    ]


_lib_handle = None


def library_path() -> str:
    return _build.LIB


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not _build.lib_is_current():
            # missing, or built from other sources: rebuild, and fail loudly
            # where no compiler is available rather than run a stale binary
            try:
                _build.build()
            except Exception as e:
                raise RuntimeError(f"{_build.LIB} is missing or older than its sources, and "
                                   f"rebuilding it failed: {e}") from e
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.POINTER(_Args)
        lib.paged_attn_fwd.restype = ctypes.c_int
        lib.paged_attn_fwd.argtypes = [P, ctypes.c_void_p]
        lib.paged_attn_fwd_noalloc.restype = ctypes.c_int
        lib.paged_attn_fwd_noalloc.argtypes = [P, ctypes.c_void_p]
        lib.paged_kv_append.restype = ctypes.c_int
        lib.paged_kv_append.argtypes = [P, ctypes.c_void_p]
        lib.paged_attn_workspace_size.restype = ctypes.c_size_t
        lib.paged_attn_workspace_size.argtypes = [P]
        lib.paged_attn_splits_for.restype = ctypes.c_int32
        lib.paged_attn_splits_for.argtypes = [P]
        lib.paged_attn_num_splits.restype = ctypes.c_int32
        lib.paged_attn_num_splits.argtypes = [ctypes.c_int32] * 8
        lib.paged_attn_status_string.restype = ctypes.c_char_p
        lib.paged_attn_status_string.argtypes = [ctypes.c_int32]
        _lib_handle = lib
    return _lib_handle


def paged_attn_status_string(status: int) -> str:
    return _lib().paged_attn_status_string(int(status)).decode()


def paged_attn_num_splits(batch, total_q, num_heads_q, num_heads_kv, head_dim, max_seqlen_q,
                          max_seqlen_k, num_cus) -> int:
    return int(_lib().paged_attn_num_splits(batch, total_q, num_heads_q, num_heads_kv, head_dim,
                                            max_seqlen_q, max_seqlen_k, num_cus))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(name, t, dtype=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_rows(name, t, dtype):
    """q / k_new / v_new: [tokens, heads, head_dim] with heads and head_dim dense;
    the token stride may be larger (a view into a fused QKV output).  Returns
    the row stride to pass (0 when dense)."""
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [tokens, heads, head_dim] with heads and head_dim dense")
    if t.is_contiguous():
        return 0
    return int(t.stride(0))


def _shape(name, t, want):
    """Raise unless tensor `t` has shape `want` (a tuple; None entries match anything)."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        raise ValueError(f"{name} has shape {list(got)}, expected "
                         f"{['*' if w is None else w for w in want]}")


def _check_same_gpu(**tensors):
    """Every given tensor lives on one GPU (the kernels dereference them all
    there): a host tensor or one on another device would be read through a
    wrong address."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _check_cache(k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, head_dim):
    """Shapes shared by the forward call and the append: pools, table, metadata.
    Returns (batch, num_heads_kv)."""
    if cache_seqlens.dim() != 1 or cache_seqlens.shape[0] < 1:
        raise ValueError("cache_seqlens must be [batch] with batch >= 1")
    batch = cache_seqlens.shape[0]
    _shape("cu_seqlens_q", cu_seqlens_q, (batch + 1,))
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [num_pages, page_size, num_heads_kv, head_dim] "
                         "(or [batch, alloc, num_heads_kv, head_dim] without a block table)")
    _shape("v_cache", v_cache, tuple(k_cache.shape))
    if k_cache.shape[3] != head_dim:
        raise ValueError(f"k_cache head_dim {k_cache.shape[3]} != {head_dim}")
    if block_table is not None:
        _shape("block_table", block_table, (batch, None))
    elif k_cache.shape[0] != batch:
        raise ValueError("contiguous k_cache / v_cache must be [batch, alloc, num_heads_kv, "
                         f"head_dim]: leading size {k_cache.shape[0]} != batch {batch}")
    return batch, k_cache.shape[2]


def _set_rotary(a: _Args, rotary_cos, rotary_sin, rotary_interleaved, dtype) -> None:
    """Fill the rotary fields: tables [rows, rotary_dim / 2] in the element type."""
    if (rotary_cos is None) != (rotary_sin is None):
        raise ValueError("rotary_cos and rotary_sin go together")
    if rotary_cos is None:
        return
    _check_dev("rotary_cos", rotary_cos, dtype)
    _check_dev("rotary_sin", rotary_sin, dtype)
    if rotary_cos.dim() != 2 or rotary_cos.shape != rotary_sin.shape:
        raise ValueError("rotary_cos / rotary_sin must both be [rows, rotary_dim / 2]")
    a.rotary_cos = _ptr(rotary_cos)
    a.rotary_sin = _ptr(rotary_sin)
    a.rotary_rows = rotary_cos.shape[0]
    a.rotary_dim = 2 * rotary_cos.shape[1]
    a.rotary_interleaved = int(bool(rotary_interleaved))


def make_args(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, *, max_seqlen_q,
              max_seqlen_k=0, k_new=None, v_new=None, causal=False, num_splits=0,
              softmax_scale=None, out=None, softmax_lse=None, workspace=None, rotary_cos=None,
              rotary_sin=None, rotary_interleaved=False) -> _Args:
    """Fill a ``pa_fwd_args`` from tensors (shapes read from the tensors).

    Every shape the kernels rely on is checked here, then that every tensor
    is on one GPU; a mismatch raises before anything reaches the library.
    ``out`` / ``softmax_lse`` may be None only for sizing queries."""
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError("q must be float16 or bfloat16")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        _check_dev(name, t, dt)
    q_stride = _check_rows("q", q, dt)
    kn_stride = _check_rows("k_new", k_new, dt)
    vn_stride = _check_rows("v_new", v_new, dt)
    for name, t in (("block_table", block_table), ("cache_seqlens", cache_seqlens),
                    ("cu_seqlens_q", cu_seqlens_q)):
        _check_dev(name, t, torch.int32)
    _check_dev("softmax_lse", softmax_lse, torch.float32)
    _check_dev("workspace", workspace)
    total_q, hq, d = q.shape
    batch, hkv = _check_cache(k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, d)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        _shape("k_new", k_new, (total_q, hkv, d))
        _shape("v_new", v_new, (total_q, hkv, d))
    if out is not None:
        _shape("out", out, (total_q, hq, d))
    if softmax_lse is not None:
        _shape("softmax_lse", softmax_lse, (total_q, hq))
    _check_same_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                    cache_seqlens=cache_seqlens, cu_seqlens_q=cu_seqlens_q, k_new=k_new,
                    v_new=v_new, out=out, softmax_lse=softmax_lse, workspace=workspace,
                    rotary_cos=rotary_cos, rotary_sin=rotary_sin)
    a = _Args()
    a.dtype = _DTYPE_CODE[dt]
    a.batch = batch
    a.total_q = total_q
    a.max_seqlen_q = int(max_seqlen_q)
    a.max_seqlen_k = int(max_seqlen_k)
    a.num_heads_q = hq
    a.num_heads_kv = hkv
    a.head_dim = d
    if block_table is not None:
        a.page_size = k_cache.shape[1]
        a.num_pages = k_cache.shape[0]
        a.max_pages_per_seq = block_table.shape[1]
        a.contig_alloc = 0
    else:
        a.contig_alloc = k_cache.shape[1]
    a.causal = int(bool(causal))
    a.num_splits = int(num_splits)
    a.softmax_scale = float(softmax_scale) if softmax_scale is not None else 0.0
    a.reserved0 = 0
    a.q = _ptr(q)
    a.k_cache = _ptr(k_cache)
    a.v_cache = _ptr(v_cache)
    a.block_table = _ptr(block_table)
    a.cache_seqlens = _ptr(cache_seqlens)
    a.cu_seqlens_q = _ptr(cu_seqlens_q)
    a.k_new = _ptr(k_new)
    a.v_new = _ptr(v_new)
    a.out = _ptr(out)
    a.softmax_lse = _ptr(softmax_lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _set_rotary(a, rotary_cos, rotary_sin, rotary_interleaved, dt)
    a.q_row_stride, a.k_new_row_stride, a.v_new_row_stride = q_stride, kn_stride, vn_stride
    return a


def paged_attn_workspace_size(args: _Args) -> int:
    return int(_lib().paged_attn_workspace_size(ctypes.byref(args)))


def paged_attn_splits_for(args: _Args) -> int:
    return int(_lib().paged_attn_splits_for(ctypes.byref(args)))


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


_aux_streams = {}


def default_aux_stream(device) -> torch.cuda.Stream:
    """The binding's second stream for mixed batches on `device` (one per
    device, default priority, created on first use and kept by the binding)."""
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    s = _aux_streams.get(idx)
    if s is None:
        s = torch.cuda.Stream(device=idx)
        _aux_streams[idx] = s
    return s


def paged_attn_fwd(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, *,
                   max_seqlen_q: int, max_seqlen_k: int = 0, k_new=None, v_new=None,
                   causal: bool = False, num_splits: int = 0, softmax_scale=None, out=None,
                   softmax_lse=None, workspace=None, rotary_cos=None, rotary_sin=None,
                   rotary_interleaved: bool = False, stream=None,
                   aux_stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Paged attention forward (with optional in-call append of k_new/v_new).

    q [total_q, Hq, D]; k_cache/v_cache [num_pages, page_size, Hkv, D] (or
    [batch, alloc, Hkv, D] with ``block_table=None``); block_table [batch,
    width] int32; cache_seqlens [batch] int32; cu_seqlens_q [batch+1] int32.
    ``max_seqlen_q`` must bound every q_len on the host side (no device read).
    ``rotary_cos`` / ``rotary_sin`` [rows, rotary_dim / 2] (element type) turn
    on the fused rotary embedding of q and k_new.
    Everything is queued on ``stream`` (default: torch's current stream).  A
    batch that can mix decode-mode and prefill-mode sequences runs its prefill
    units and then its decode units there; with ``aux_stream`` (a stream, or
    "auto" for the binding's own second stream of the device) the decode units
    run on it instead, concurrently, forked from ``stream`` and joined back
    into it by the call, so later work on ``stream`` sees the whole result.  Tensors the call allocates (out, softmax_lse, workspace when not
    given) are allocated on ``stream``, so the caching allocator does not hand
    them out again before the kernels queued there have finished.
    Returns (out [total_q, Hq, D], softmax_lse [total_q, Hq] fp32).
    """
    # every check first: nothing is allocated or launched for bad arguments
    args = make_args(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q,
                     max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, k_new=k_new,
                     v_new=v_new, causal=causal, num_splits=num_splits,
                     softmax_scale=softmax_scale, out=out, softmax_lse=softmax_lse,
                     workspace=workspace, rotary_cos=rotary_cos, rotary_sin=rotary_sin,
                     rotary_interleaved=rotary_interleaved)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    aux = default_aux_stream(q.device) if isinstance(aux_stream, str) and aux_stream == "auto" \
        else aux_stream
    args.aux_stream = None if aux is None else aux.cuda_stream
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty_like(q, memory_format=torch.contiguous_format)
            args.out = out.data_ptr()
        if softmax_lse is None:
            softmax_lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
            args.softmax_lse = softmax_lse.data_ptr()
        if workspace is None:
            need = paged_attn_workspace_size(args)
            if need > 0:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
                args.workspace = workspace.data_ptr()
                args.workspace_bytes = need
    st = _lib().paged_attn_fwd(ctypes.byref(args), ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise PagedAttnError(st, "paged_attn_fwd")
    return out, softmax_lse


def paged_attn_fwd_noalloc(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, *,
                           out, softmax_lse, max_seqlen_q: int, max_seqlen_k: int = 0,
                           k_new=None, v_new=None, causal: bool = False, num_splits: int = 0,
                           softmax_scale=None, rotary_cos=None, rotary_sin=None,
                           rotary_interleaved: bool = False, stream=None) -> None:
    """The allocation-free entry point: as paged_attn_fwd, with the caller's
    ``out`` / ``softmax_lse`` (required) and the library's static split-KV
    scratch in place of a workspace; neither the binding nor the library
    allocates anything, and every launch of a mixed batch runs on ``stream``
    (none is forked onto a second stream).  Calls that overlap on one GPU
    share the scratch and must be serialised."""
    if out is None or softmax_lse is None:
        raise ValueError("paged_attn_fwd_noalloc writes into the caller's out and softmax_lse")
    args = make_args(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q,
                     max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, k_new=k_new,
                     v_new=v_new, causal=causal, num_splits=num_splits,
                     softmax_scale=softmax_scale, out=out, softmax_lse=softmax_lse,
                     rotary_cos=rotary_cos, rotary_sin=rotary_sin,
                     rotary_interleaved=rotary_interleaved)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = _lib().paged_attn_fwd_noalloc(ctypes.byref(args), ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise PagedAttnError(st, "paged_attn_fwd_noalloc")


def paged_kv_append(k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, k_new, v_new, *,
                    max_seqlen_q: int, rotary_cos=None, rotary_sin=None,
                    rotary_interleaved: bool = False, stream=None) -> None:
    """Write k_new/v_new rows at positions cache_seqlens[b] + i (bit copy; keys
    rotated at those positions first when rotary tables are given)."""
    dt = k_cache.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError("k_cache must be float16 or bfloat16")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check_dev(name, t, dt)
    for name, t in (("block_table", block_table), ("cache_seqlens", cache_seqlens),
                    ("cu_seqlens_q", cu_seqlens_q)):
        _check_dev(name, t, torch.int32)
    if k_new is None or v_new is None:
        raise ValueError("paged_kv_append needs k_new and v_new")
    kn_stride = _check_rows("k_new", k_new, dt)
    vn_stride = _check_rows("v_new", v_new, dt)
    d = k_new.shape[2]
    batch, hkv = _check_cache(k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, d)
    _shape("k_new", k_new, (k_new.shape[0], hkv, d))
    _shape("v_new", v_new, tuple(k_new.shape))
    _check_same_gpu(k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                    cache_seqlens=cache_seqlens, cu_seqlens_q=cu_seqlens_q, k_new=k_new,
                    v_new=v_new, rotary_cos=rotary_cos, rotary_sin=rotary_sin)
    a = _Args()
    a.dtype = _DTYPE_CODE[dt]
    a.batch = batch
    a.total_q = k_new.shape[0]
    a.max_seqlen_q = int(max_seqlen_q)
    a.num_heads_q = hkv
    a.num_heads_kv = hkv
    a.head_dim = d
    if block_table is not None:
        a.page_size = k_cache.shape[1]
        a.num_pages = k_cache.shape[0]
        a.max_pages_per_seq = block_table.shape[1]
    else:
        a.contig_alloc = k_cache.shape[1]
    a.k_cache = _ptr(k_cache)
    a.v_cache = _ptr(v_cache)
    a.block_table = _ptr(block_table)
    a.cache_seqlens = _ptr(cache_seqlens)
    a.cu_seqlens_q = _ptr(cu_seqlens_q)
    a.k_new = _ptr(k_new)
    a.v_new = _ptr(v_new)
    a.k_new_row_stride, a.v_new_row_stride = kn_stride, vn_stride
    _set_rotary(a, rotary_cos, rotary_sin, rotary_interleaved, dt)
    st = _lib().paged_kv_append(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream)))
    if st != 0:
        raise PagedAttnError(st, "paged_kv_append")
