"""Paged KV-cache attention for MI355X (gfx950): Python binding of libpagedkv.so.

Thin argument marshalling over the C ABI declared in include/pagedkv.h: torch
tensors are checked for dtype, device and contiguity, and passed as raw device
pointers together with torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, importing this package raises ImportError.

    kv_store(key, value, slot_mapping, k_cache, v_cache)
    paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale, ...)
    paged_prefill(q, k_cache, v_cache, block_tables, cu_seqlens_q, cu_seqlens_k, scale, ...)
    paged_prefill_store(q, key, value, k_cache, v_cache, block_tables, cu_seqlens_q, ...)
    paged_prefill_decode(q, k_cache, v_cache, block_tables, cu_seqlens_q, cu_seqlens_k, ...)
    BlockManager(num_blocks, block_size)   host-side block allocation with prefix caching
"""
from __future__ import annotations

import ctypes
import functools
import os
import weakref
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "PagedKVError", "version", "kv_store", "paged_decode", "paged_decode_store",
    "paged_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "paged_prefill", "paged_prefill_store", "paged_prefill_decode",
    "decode_plan", "decode_workspace_size", "BlockManager", "check_indices",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python paged_kv_cache_236_amd/build.py` "
        "(or __graft_entry__.build()); there is no non-HIP implementation")

_lib = ctypes.CDLL(LIB_PATH)

_i32 = ctypes.c_int32
_p = ctypes.c_void_p
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_lib.pk_version.restype = ctypes.c_char_p
_lib.pk_version.argtypes = []
_lib.pk_status_string.restype = ctypes.c_char_p
_lib.pk_status_string.argtypes = [ctypes.c_int]
_lib.pk_last_error_message.restype = ctypes.c_char_p
_lib.pk_last_error_message.argtypes = []
_lib.pk_kv_store.restype = ctypes.c_int
_lib.pk_kv_store.argtypes = [_p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _p]
_lib.pk_paged_decode_plan.restype = ctypes.c_int
_lib.pk_paged_decode_plan.argtypes = [_i32, _i32, _i32, _i32, _i32,
                                      ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
_lib.pk_paged_decode_workspace_size.restype = _sz
_lib.pk_paged_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
_lib.pk_paged_decode.restype = ctypes.c_int
_lib.pk_paged_decode.argtypes = [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p, _i32,
                                 _i32, _i32, _f32, _i32, _i32, _p, _sz, _p]
_lib.pk_paged_decode_noalloc.restype = ctypes.c_int
_lib.pk_paged_decode_noalloc.argtypes = [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p, _i32,
                                         _i32, _i32, _f32, _i32, _i32, _p]
_lib.pk_paged_decode_store.restype = ctypes.c_int
_lib.pk_paged_decode_store.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p,
                                       _i32, _i32, _i32, _f32, _i32, _i32, _p, _sz, _p]
_lib.pk_paged_prefill.restype = ctypes.c_int
_lib.pk_paged_prefill.argtypes = [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p, _p,
                                  _i32, _i32, _i32, _i32, _f32, _i32, _p]
_lib.pk_paged_prefill_store.restype = ctypes.c_int
_lib.pk_paged_prefill_store.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32,
                                        _p, _p, _i32, _i32, _i32, _i32, _f32, _i32, _p]
_lib.pk_paged_prefill_decode.restype = ctypes.c_int
_lib.pk_paged_prefill_decode.argtypes = [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p, _p,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]
_lib.pk_check_indices_workspace_size.restype = _sz
_lib.pk_check_indices_workspace_size.argtypes = [_i32, _i32]
_lib.pk_check_indices.restype = ctypes.c_int
_lib.pk_check_indices.argtypes = [_p, _i32, _p, _i32, _i32, _p, _p, _p, _i32, _i32, _p, _p, _sz, _p]
_i64 = ctypes.c_int64
_pi32 = ctypes.POINTER(_i32)
for _name, _args in (
        ("pk_bm_create", [_i32, _i32, ctypes.POINTER(_p)]),
        ("pk_bm_num_free_blocks", [_p, _pi32]),
        ("pk_bm_block_info", [_p, _i32, _pi32, _pi32]),
        ("pk_bm_allocate", [_p, _i64, _p, _i32, _pi32]),
        ("pk_bm_append", [_p, _i64, _i32]),
        ("pk_bm_commit", [_p, _pi32]),
        ("pk_bm_free", [_p, _i64]),
        ("pk_bm_seq_info", [_p, _i64, _pi32, _pi32, _pi32]),
        ("pk_bm_prepare", [_p, _p, _i32, _p, _i32, _p, _p, _p, _p])):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = _args
_lib.pk_bm_destroy.restype = None
_lib.pk_bm_destroy.argtypes = [_p]


class PagedKVError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, message: str):
        self.status = status
        name = _lib.pk_status_string(status).decode()
        super().__init__(f"{name}: {message}")


def _check(status: int) -> None:
    if status != 0:
        raise PagedKVError(status, _lib.pk_last_error_message().decode())


def version() -> str:
    return _lib.pk_version().decode()


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, device=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    """torch's current HIP stream on `device`, as a raw handle."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_blocks, block_size, num_kv_heads, head_dim]")
    return tuple(int(x) for x in k_cache.shape)


def kv_store(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
             k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Store key/value [num_tokens, num_kv_heads, head_dim] (bf16) into the
    caches at slot_mapping (int32 [num_tokens]; -1 skips a token)."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    n = int(slot_mapping.numel())
    if key.shape != (n, hkv, d) or value.shape != (n, hkv, d):
        raise ValueError(f"key/value must be [{n}, {hkv}, {d}]")
    _check(_lib.pk_kv_store(
        _dev(key, "key", torch.bfloat16, dev), _dev(value, "value", torch.bfloat16, dev),
        _dev(slot_mapping, "slot_mapping", torch.int32, dev), n,
        _dev(k_cache, "k_cache", torch.bfloat16, dev), _dev(v_cache, "v_cache", torch.bfloat16, dev),
        nb, bs, hkv, d, _stream(dev)))


def decode_plan(num_seqs: int, num_kv_heads: int, max_context_len: int,
                sliding_window: int = 0, partition_size: int = 0):
    """(partition_size, partition slots per sequence) that paged_decode uses."""
    ps, nparts = _i32(), _i32()
    _check(_lib.pk_paged_decode_plan(num_seqs, num_kv_heads, max_context_len, sliding_window,
                                     partition_size, ctypes.byref(ps), ctypes.byref(nparts)))
    return ps.value, nparts.value


@functools.lru_cache(maxsize=1024)
def _workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                    sliding_window, partition_size):
    n = _lib.pk_paged_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            max_context_len, sliding_window, partition_size)
    if n == 0:
        msg = _lib.pk_last_error_message().decode()
        if msg:
            return msg
    return int(n)


def decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          max_context_len: int, sliding_window: int = 0,
                          partition_size: int = 0) -> int:
    """Workspace bytes paged_decode needs (a pure function of its arguments, so
    the answer is cached)."""
    n = _workspace_size(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                        int(max_context_len), int(sliding_window), int(partition_size))
    if isinstance(n, str):
        raise PagedKVError(1, n)
    return n


_workspaces = {}


def _workspace(device, nbytes: int) -> Optional[torch.Tensor]:
    """A grow-only per-device scratch buffer for the split-K partials."""
    if nbytes == 0:
        return None
    key = (device.type, device.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _decode_common(q, k_cache, v_cache, block_tables, context_lens, sliding_window,
                   max_context_len, out, partition_size, workspace):
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    nseq, hq, qd = (int(x) for x in q.shape)
    if qd != d:
        raise ValueError("q and cache head_dim differ")
    if block_tables.dim() != 2 or block_tables.shape[0] != nseq or context_lens.shape != (nseq,):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and context_lens [num_seqs]")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if nseq else 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    dev = q.device
    need = decode_workspace_size(nseq, hq, hkv, d, max_context_len, sliding_window, partition_size)
    if workspace is None:
        workspace = _workspace(dev, need)
    ws_ptr = _dev(workspace, "workspace", torch.uint8, dev) if workspace is not None else None
    ws_bytes = int(workspace.numel()) if workspace is not None else 0
    return (nb, bs, hkv, d, nseq, hq, max_context_len, out, ws_ptr, ws_bytes)


def paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, *,
                 sliding_window: int = 0, max_context_len: Optional[int] = None,
                 out: Optional[torch.Tensor] = None, partition_size: int = 0,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention: q [num_seqs, num_q_heads, 128] bf16 -> out (same shape).

    max_context_len defaults to context_lens.max() (a device-to-host sync);
    pass it to keep the call asynchronous.
    """
    dev = q.device
    nb, bs, hkv, d, nseq, hq, mcl, out, ws_ptr, ws_bytes = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, sliding_window, max_context_len, out,
        partition_size, workspace)
    _check(_lib.pk_paged_decode(
        _dev(out, "out", torch.bfloat16, dev), _dev(q, "q", torch.bfloat16, dev),
        _dev(k_cache, "k_cache", torch.bfloat16, dev), _dev(v_cache, "v_cache", torch.bfloat16, dev),
        nb, bs, hkv, d,
        _dev(block_tables, "block_tables", torch.int32, dev), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", torch.int32, dev), nseq, hq, mcl,
        float(scale), sliding_window, partition_size, ws_ptr, ws_bytes, _stream(dev)))
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20   # PK_NOALLOC_SCRATCH_BYTES in pagedkv.h


def paged_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, *,
                         max_context_len: int, out: torch.Tensor, sliding_window: int = 0,
                         partition_size: int = 0) -> torch.Tensor:
    """paged_decode for callers that cannot allocate device memory: the
    split-K partials use the library's static per-GPU scratch
    (NOALLOC_SCRATCH_BYTES), so neither this call nor the library allocates.
    `out` and `max_context_len` are required (no allocation, no device sync).
    Calls that overlap on one GPU share the scratch and race: keep them on one
    stream."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    nseq, hq, qd = (int(x) for x in q.shape)
    if qd != d:
        raise ValueError("q and cache head_dim differ")
    if block_tables.dim() != 2 or block_tables.shape[0] != nseq or context_lens.shape != (nseq,):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and context_lens [num_seqs]")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    dev = q.device
    _check(_lib.pk_paged_decode_noalloc(
        _dev(out, "out", torch.bfloat16, dev), _dev(q, "q", torch.bfloat16, dev),
        _dev(k_cache, "k_cache", torch.bfloat16, dev), _dev(v_cache, "v_cache", torch.bfloat16, dev),
        nb, bs, hkv, d,
        _dev(block_tables, "block_tables", torch.int32, dev), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", torch.int32, dev), nseq, hq, int(max_context_len),
        float(scale), sliding_window, partition_size, _stream(dev)))
    return out


def paged_decode_store(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                       context_lens: torch.Tensor, scale: float, *, sliding_window: int = 0,
                       max_context_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
                       partition_size: int = 0,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Store the new token k_new/v_new [num_seqs, num_kv_heads, 128] at position
    context_lens-1 of each sequence and run decode attention, in one launch."""
    dev = q.device
    nb, bs, hkv, d, nseq, hq, mcl, out, ws_ptr, ws_bytes = _decode_common(
        q, k_cache, v_cache, block_tables, context_lens, sliding_window, max_context_len, out,
        partition_size, workspace)
    if k_new.shape != (nseq, hkv, d) or v_new.shape != (nseq, hkv, d):
        raise ValueError(f"k_new/v_new must be [{nseq}, {hkv}, {d}]")
    _check(_lib.pk_paged_decode_store(
        _dev(out, "out", torch.bfloat16, dev), _dev(q, "q", torch.bfloat16, dev),
        _dev(k_new, "k_new", torch.bfloat16, dev), _dev(v_new, "v_new", torch.bfloat16, dev),
        _dev(k_cache, "k_cache", torch.bfloat16, dev), _dev(v_cache, "v_cache", torch.bfloat16, dev),
        nb, bs, hkv, d,
        _dev(block_tables, "block_tables", torch.int32, dev), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", torch.int32, dev), nseq, hq, mcl,
        float(scale), sliding_window, partition_size, ws_ptr, ws_bytes, _stream(dev)))
    return out


def paged_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_tables: torch.Tensor, cu_seqlens_q: torch.Tensor,
                  cu_seqlens_k: torch.Tensor, scale: float, *, max_seqlen_q: int,
                  sliding_window: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Varlen causal prefill: q [total_q, num_q_heads, 128] bf16 -> out (same shape)."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [total_q, num_q_heads, head_dim]")
    total_q, hq, qd = (int(x) for x in q.shape)
    if qd != d:
        raise ValueError("q and cache head_dim differ")
    nseq = int(cu_seqlens_q.numel()) - 1
    if nseq < 0 or cu_seqlens_k.shape != cu_seqlens_q.shape or block_tables.dim() != 2 \
            or block_tables.shape[0] != nseq:
        raise ValueError("cu_seqlens_q/k must be [num_seqs+1] and block_tables [num_seqs, max_blocks]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _check(_lib.pk_paged_prefill(
        _dev(out, "out", torch.bfloat16, dev), _dev(q, "q", torch.bfloat16, dev),
        _dev(k_cache, "k_cache", torch.bfloat16, dev), _dev(v_cache, "v_cache", torch.bfloat16, dev),
        nb, bs, hkv, d,
        _dev(block_tables, "block_tables", torch.int32, dev), int(block_tables.shape[1]),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev),
        nseq, total_q, int(max_seqlen_q), hq, float(scale), sliding_window, _stream(dev)))
    return out


def paged_prefill_store(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                        cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, scale: float, *,
                        max_seqlen_q: int, sliding_window: int = 0,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Store the new tokens key/value [total_q, num_kv_heads, 128] at their
    positions (from block_tables) and run the varlen prefill, in one launch."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [total_q, num_q_heads, head_dim]")
    total_q, hq, qd = (int(x) for x in q.shape)
    if qd != d:
        raise ValueError("q and cache head_dim differ")
    if key.shape != (total_q, hkv, d) or value.shape != (total_q, hkv, d):
        raise ValueError(f"key/value must be [{total_q}, {hkv}, {d}]")
    nseq = int(cu_seqlens_q.numel()) - 1
    if nseq < 0 or cu_seqlens_k.shape != cu_seqlens_q.shape or block_tables.dim() != 2 \
            or block_tables.shape[0] != nseq:
        raise ValueError("cu_seqlens_q/k must be [num_seqs+1] and block_tables [num_seqs, max_blocks]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _check(_lib.pk_paged_prefill_store(
        _dev(out, "out", torch.bfloat16, dev), _dev(q, "q", torch.bfloat16, dev),
        _dev(key, "key", torch.bfloat16, dev), _dev(value, "value", torch.bfloat16, dev),
        _dev(k_cache, "k_cache", torch.bfloat16, dev), _dev(v_cache, "v_cache", torch.bfloat16, dev),
        nb, bs, hkv, d,
        _dev(block_tables, "block_tables", torch.int32, dev), int(block_tables.shape[1]),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev),
        nseq, total_q, int(max_seqlen_q), hq, float(scale), sliding_window, _stream(dev)))
    return out


def paged_prefill_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         cu_seqlens_k: torch.Tensor, scale: float, *, num_decode_seqs: int,
                         max_seqlen_q: int, max_decode_context_len: int, sliding_window: int = 0,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A mixed batch whose first num_decode_seqs sequences have one new token
    each: those on the decode kernel, the rest on the varlen prefill kernel."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [total_q, num_q_heads, head_dim]")
    total_q, hq, qd = (int(x) for x in q.shape)
    if qd != d:
        raise ValueError("q and cache head_dim differ")
    nseq = int(cu_seqlens_q.numel()) - 1
    if nseq < 0 or cu_seqlens_k.shape != cu_seqlens_q.shape or block_tables.dim() != 2 \
            or block_tables.shape[0] != nseq:
        raise ValueError("cu_seqlens_q/k must be [num_seqs+1] and block_tables [num_seqs, max_blocks]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    nd = int(num_decode_seqs)
    need = decode_workspace_size(nd, hq, hkv, d, int(max_decode_context_len), sliding_window) \
        if nd > 0 else 0
    if workspace is None:
        workspace = _workspace(dev, need)
    ws_ptr = _dev(workspace, "workspace", torch.uint8, dev) if workspace is not None else None
    ws_bytes = int(workspace.numel()) if workspace is not None else 0
    _check(_lib.pk_paged_prefill_decode(
        _dev(out, "out", torch.bfloat16, dev), _dev(q, "q", torch.bfloat16, dev),
        _dev(k_cache, "k_cache", torch.bfloat16, dev), _dev(v_cache, "v_cache", torch.bfloat16, dev),
        nb, bs, hkv, d,
        _dev(block_tables, "block_tables", torch.int32, dev), int(block_tables.shape[1]),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev),
        nseq, nd, total_q, int(max_seqlen_q), int(max_decode_context_len), hq, float(scale),
        sliding_window, ws_ptr, ws_bytes, _stream(dev)))
    return out


PK_ERR_INDEX = 5
CHECK_FIELDS = ("slots_out_of_range", "repeated_slots", "bad_table_entries", "bad_lengths")


def check_indices(k_cache: torch.Tensor, *, slot_mapping: Optional[torch.Tensor] = None,
                  block_tables: Optional[torch.Tensor] = None,
                  context_lens: Optional[torch.Tensor] = None,
                  cu_seqlens_q: Optional[torch.Tensor] = None,
                  cu_seqlens_k: Optional[torch.Tensor] = None, raise_on_error: bool = True):
    """Checked mode: validate the index arrays on the device against the cache
    geometry of k_cache [num_blocks, block_size, Hkv, d]; returns the violation
    counts (a dict), raising PagedKVError(PK_ERR_INDEX) when any is non-zero
    and raise_on_error is set.  Synchronises the current stream."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [num_blocks, block_size, num_kv_heads, head_dim]")
    nb, bs = int(k_cache.shape[0]), int(k_cache.shape[1])
    dev = k_cache.device
    nt = int(slot_mapping.numel()) if slot_mapping is not None else 0
    if block_tables is not None:
        if block_tables.dim() != 2:
            raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
        nseq, mb = int(block_tables.shape[0]), int(block_tables.shape[1])
    else:
        nseq, mb = 0, 0
    opt = lambda t, name: _dev(t, name, torch.int32, dev) if t is not None else None
    counts = torch.empty(4, dtype=torch.int32, device=dev)
    ws = torch.empty(max(int(_lib.pk_check_indices_workspace_size(nb, bs)), 4), dtype=torch.uint8,
                     device=dev)
    _check(_lib.pk_check_indices(opt(slot_mapping, "slot_mapping"), nt,
                                 opt(block_tables, "block_tables"), mb, nseq,
                                 opt(context_lens, "context_lens"), opt(cu_seqlens_q, "cu_seqlens_q"),
                                 opt(cu_seqlens_k, "cu_seqlens_k"), nb, bs, counts.data_ptr(),
                                 ws.data_ptr(), int(ws.numel()), _stream(dev)))
    res = dict(zip(CHECK_FIELDS, (int(v) for v in counts.cpu().tolist())))
    if raise_on_error and any(res.values()):
        raise PagedKVError(PK_ERR_INDEX, f"index arrays violate the contract: {res}")
    return res


def _host_i32(values, name: str) -> torch.Tensor:
    t = torch.as_tensor(values, dtype=torch.int32, device="cpu").contiguous()
    if t.dim() != 1:
        raise ValueError(f"{name} must be one-dimensional")
    return t


class BlockManager:
    """Host-side KV block manager with prefix caching (pk_bm_* in pagedkv.h).

    Blocks are ids into a cache of ``num_blocks`` blocks of ``block_size``
    slots.  ``allocate`` admits a sequence and returns how many leading prompt
    tokens reuse cached blocks; ``append`` adds a generated token; ``free``
    drops a sequence; ``prepare`` returns the int32 CPU tensors one attention
    call needs (block_tables, cu_seqlens_q, cu_seqlens_k, slot_mapping);
    ``commit`` ends a step: blocks filled during it become findable only then,
    so a batch never reuses a prefix block that the same batch writes.
    """

    def __init__(self, num_blocks: int, block_size: int):
        h = _p()
        _check(_lib.pk_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h = h
        self._finalizer = weakref.finalize(self, _lib.pk_bm_destroy, h)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        """Destroy the manager now (otherwise it goes with the object)."""
        self._finalizer()
        self._h = _p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _handle(self):
        if not self._h:
            raise ValueError("BlockManager is closed")
        return self._h

    @property
    def num_free_blocks(self) -> int:
        n = _i32()
        _check(_lib.pk_bm_num_free_blocks(self._handle(), ctypes.byref(n)))
        return n.value

    def block_info(self, block: int):
        """(reference count, whether the block's content is registered)."""
        ref, cached = _i32(), _i32()
        _check(_lib.pk_bm_block_info(self._handle(), int(block), ctypes.byref(ref),
                                     ctypes.byref(cached)))
        return ref.value, bool(cached.value)

    def allocate(self, seq_id: int, tokens) -> int:
        t = _host_i32(tokens, "tokens")
        n = _i32()
        _check(_lib.pk_bm_allocate(self._handle(), int(seq_id), t.data_ptr(), int(t.numel()),
                                   ctypes.byref(n)))
        return n.value

    def append(self, seq_id: int, token: int) -> None:
        _check(_lib.pk_bm_append(self._handle(), int(seq_id), int(token)))

    def commit(self) -> int:
        """Make the blocks filled since the last commit findable by later
        ``allocate`` calls; call it once the step that stores their K/V has
        been enqueued.  Returns how many blocks became findable."""
        n = _i32()
        _check(_lib.pk_bm_commit(self._handle(), ctypes.byref(n)))
        return n.value

    def free(self, seq_id: int) -> None:
        _check(_lib.pk_bm_free(self._handle(), int(seq_id)))

    def seq_info(self, seq_id: int):
        """(tokens, blocks, cached leading tokens) of a sequence."""
        a, b, c = _i32(), _i32(), _i32()
        _check(_lib.pk_bm_seq_info(self._handle(), int(seq_id), ctypes.byref(a), ctypes.byref(b),
                                   ctypes.byref(c)))
        return a.value, b.value, c.value

    def prepare(self, seq_ids, num_new, max_blocks_per_seq: int):
        """block_tables [B, max_blocks_per_seq], cu_seqlens_q [B+1], cu_seqlens_k [B+1]
        and slot_mapping [sum(num_new)], all int32 CPU tensors."""
        ids = torch.as_tensor(seq_ids, dtype=torch.int64, device="cpu").contiguous()
        nn = _host_i32(num_new, "num_new")
        b = int(ids.numel())
        if ids.dim() != 1 or nn.numel() != b:
            raise ValueError("seq_ids and num_new must be one-dimensional and equally long")
        tables = torch.empty(b, int(max_blocks_per_seq), dtype=torch.int32)
        cu_q = torch.empty(b + 1, dtype=torch.int32)
        cu_k = torch.empty(b + 1, dtype=torch.int32)
        slots = torch.empty(max(int(nn.sum()), 0), dtype=torch.int32)
        _check(_lib.pk_bm_prepare(self._handle(), ids.data_ptr(), b, nn.data_ptr(),
                                  int(max_blocks_per_seq), tables.data_ptr(), cu_q.data_ptr(),
                                  cu_k.data_ptr(), slots.data_ptr()))
        return tables, cu_q, cu_k, slots
