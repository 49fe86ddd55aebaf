"""Thin Python binding of libnvpaged.so.

The functions carry the C entry points' names and only marshal arguments:
device tensors become raw pointers, host arrays become int32 buffers, and the
current torch stream becomes the hipStream_t.  Every step of the path runs in
the HIP library; nothing here computes attention or copies cache rows.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import numpy as np
import torch

from . import _native

NV_OK = 0
NV_F32 = 0
NV_BF16 = 1

_DTYPES = {torch.float32: NV_F32, torch.bfloat16: NV_BF16}


class NvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _native.load().nv_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")


def _check(fn: str, status: int):
    if status != NV_OK:
        raise NvError(fn, status)


def nv_status_string(status: int) -> str:
    return _native.load().nv_status_string(status).decode()


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _dev(t: torch.Tensor, name: str, contiguous: bool = True) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_native.c_i32p)


# ---------------------------------------------------------------------------
# store_kvcache
# ---------------------------------------------------------------------------

def _store_call(k, v, k_cache, v_cache, slot_mapping, stream):
    nb, bs, hkv, d = k_cache.shape
    n = k.shape[0]
    for name, t in (("k", k), ("v", v)):
        if t.shape[1:] != (hkv, d) or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{name} must be [N, {hkv}, {d}] with contiguous heads")
    if slot_mapping.dtype != torch.int32 or slot_mapping.numel() != n:
        raise ValueError("slot_mapping must be int32 with one entry per row")
    args = (_dev(k, "k", False), _dev(v, "v", False), k.stride(0), v.stride(0),
            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping"),
            n, hkv, d, nb, bs, _dtype_code(k_cache), _stream(stream, k_cache.device))
    return _native.load().nv_store_kvcache, args


def nv_store_kvcache(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """k, v: [N, Hkv, D] (rows may be strided, heads and dims contiguous);
    caches: [num_blocks, block_size, Hkv, D]; slot_mapping: int32 [N] on the device."""
    fn, args = _store_call(k, v, k_cache, v_cache, slot_mapping, stream)
    _check("nv_store_kvcache", fn(*args))


def _prepared(name, fn, args, keep):
    """A callable that repeats one C call with arguments converted to ctypes once."""
    cargs = tuple(a if a is None else conv(a) for a, conv in zip(args, fn.argtypes))

    def launch(_keep=keep):
        st = fn(*cargs)
        if st != NV_OK:
            raise NvError(name, st)
    return launch


def prepare_store_kvcache(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None):
    """nv_store_kvcache with its arguments validated and marshalled once: returns a
    callable that enqueues the same store again (buffers refilled in place).  The
    callable keeps the tensors alive; the stream is the one current at preparation."""
    fn, args = _store_call(k, v, k_cache, v_cache, slot_mapping, stream)
    return _prepared("nv_store_kvcache", fn, args, (k, v, k_cache, v_cache, slot_mapping))


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def nv_paged_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int,
                                   head_dim: int, max_context_len: int) -> int:
    return int(_native.load().nv_paged_decode_workspace_size(
        batch, num_q_heads, num_kv_heads, head_dim, max_context_len))


_ws_cache = {}
_NO_WORKSPACE = object()   # marks a call that takes no workspace at all


def decode_workspace(device, nbytes: int, stream=None) -> Optional[torch.Tensor]:
    """A scratch buffer of at least nbytes for calls enqueued on ``stream`` (default: the
    device's current stream), cached per (device, stream) and reused by later calls on
    that stream, which the stream orders.  Calls on different streams get different
    buffers.  A call that needs more replaces the cached buffer; a prepared call keeps the
    buffer it was prepared with."""
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (dev, _stream(stream, dev))
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def nv_paged_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, max_context_len: int, softmax_scale: float,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    schedule: Optional[torch.Tensor] = None) -> None:
    nb, bs, hkv, d = k_cache.shape
    batch, hq = q.shape[0], q.shape[1]
    dt = _dtype_code(k_cache)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if schedule is not None and (schedule.dtype != torch.int32 or schedule.numel() != batch):
        raise ValueError("schedule must be int32 with one entry per sequence")
    if workspace is None:   # the library checks the size of a caller-provided workspace
        need = nv_paged_decode_workspace_size(batch, hq, hkv, d, max_context_len)
        workspace = decode_workspace(k_cache.device, need, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _native.load().nv_paged_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(context_lens, "context_lens"),
        _dev(schedule, "schedule") if schedule is not None else None,
        max_context_len, batch, hq, hkv, d, nb, bs,
        float(softmax_scale), dt, ws_ptr, ws_len, _stream(stream, q.device))
    _check("nv_paged_decode", st)


def _decode_store_call(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                       context_lens, max_context_len, softmax_scale, workspace, stream,
                       schedule):
    """Validate and marshal the fused store + decode arguments: (C function, args, the
    workspace tensor the arguments point into, or None)."""
    nb, bs, hkv, d = k_cache.shape
    batch, hq = q.shape[0], q.shape[1]
    dt = _dtype_code(k_cache)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.shape[0] != batch or t.shape[1:] != (hkv, d) or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{name} must be [batch, {hkv}, {d}] with contiguous heads")
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens),
                    ("slot_mapping", slot_mapping)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if schedule is not None and (schedule.dtype != torch.int32 or schedule.numel() != batch):
        raise ValueError("schedule must be int32 with one entry per sequence")
    if workspace is _NO_WORKSPACE:
        workspace = None
    elif workspace is None:   # the library checks the size of a caller-provided workspace
        need = nv_paged_decode_workspace_size(batch, hq, hkv, d, max_context_len)
        workspace = decode_workspace(k_cache.device, need, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new", False), _dev(v_new, "v_new", False),
        k_new.stride(0), v_new.stride(0), _dev(slot_mapping, "slot_mapping"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(context_lens, "context_lens"),
        _dev(schedule, "schedule") if schedule is not None else None,
        max_context_len, batch, hq, hkv, d, nb, bs, float(softmax_scale), dt, ws_ptr, ws_len,
        _stream(stream, q.device))
    return _native.load().nv_paged_decode_store, args, workspace


def nv_paged_decode_store(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                          v_new: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, block_tables: torch.Tensor,
                          context_lens: torch.Tensor, max_context_len: int,
                          softmax_scale: float, workspace: Optional[torch.Tensor] = None,
                          stream=None, schedule: Optional[torch.Tensor] = None) -> None:
    """Store this step's K/V rows and decode, fused into one launch."""
    fn, args, _ = _decode_store_call(out, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                     block_tables, context_lens, max_context_len, softmax_scale,
                                     workspace, stream, schedule)
    _check("nv_paged_decode_store", fn(*args))


def nv_paged_decode_store_noalloc(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                                  v_new: torch.Tensor, slot_mapping: torch.Tensor,
                                  k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                                  max_context_len: int, softmax_scale: float, stream=None,
                                  schedule: Optional[torch.Tensor] = None) -> None:
    """nv_paged_decode_store without a workspace: split partials go to the library's own
    per-GPU device array, so the call allocates nothing (calls on one GPU must be ordered
    on one stream)."""
    fn, args, _ = _decode_store_call(out, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                     block_tables, context_lens, max_context_len, softmax_scale,
                                     _NO_WORKSPACE, stream, schedule)
    # the same arguments minus the workspace pointer and size
    _check("nv_paged_decode_store_noalloc",
           _native.load().nv_paged_decode_store_noalloc(*args[:-3], args[-1]))


def prepare_paged_decode_store(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                               v_new: torch.Tensor, slot_mapping: torch.Tensor,
                               k_cache: torch.Tensor, v_cache: torch.Tensor,
                               block_tables: torch.Tensor, context_lens: torch.Tensor,
                               max_context_len: int, softmax_scale: float,
                               workspace: Optional[torch.Tensor] = None, stream=None,
                               schedule: Optional[torch.Tensor] = None):
    """nv_paged_decode_store with its arguments validated and marshalled once: returns a
    callable that enqueues the same launch again (for steps whose buffers are fixed and
    refilled in place, where per-call marshalling would dominate a small step).  The
    callable keeps the tensors alive, including the workspace its arguments point into
    (the cached one when ``workspace`` is None, even after the cache moves on to a larger
    buffer); the stream is the one current at preparation."""
    fn, args, ws_used = _decode_store_call(out, q, k_new, v_new, slot_mapping, k_cache,
                                           v_cache, block_tables, context_lens, max_context_len,
                                           softmax_scale, workspace, stream, schedule)
    keep = (out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens,
            ws_used, schedule)
    return _prepared("nv_paged_decode_store", fn, args, keep)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def nv_paged_prefill(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                     cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                     block_tables: torch.Tensor, softmax_scale: float, causal: bool = True,
                     stream=None, tile_schedule: Optional[torch.Tensor] = None) -> None:
    """tile_schedule: optional int32 [num_tiles, 2] (sequence, tile) pairs on the device."""
    nb, bs, hkv, d = k_cache.shape
    hq = q.shape[1]
    num_seqs = cu_seqlens_q.numel() - 1
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
                    ("block_tables", block_tables)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if tile_schedule is not None and tile_schedule.dtype != torch.int32:
        raise ValueError("tile_schedule must be int32")
    num_tiles = tile_schedule.numel() // 2 if tile_schedule is not None else 0
    st = _native.load().nv_paged_prefill(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(cu_seqlens_k, "cu_seqlens_k"),
        max_seqlen_q, max_seqlen_k, _dev(block_tables, "block_tables"), block_tables.shape[1],
        num_seqs, _dev(tile_schedule, "tile_schedule") if tile_schedule is not None else None,
        num_tiles, hq, hkv, d, nb, bs, float(softmax_scale), int(bool(causal)),
        _dtype_code(k_cache), _stream(stream, q.device))
    _check("nv_paged_prefill", st)


def nv_set_check_mode(enabled: bool) -> bool:
    """Turn check mode (device-data precondition validation before each launch) on or
    off; returns the previous setting."""
    return bool(_native.load().nv_set_check_mode(1 if enabled else 0))


def nv_check_message() -> str:
    return _native.load().nv_check_message().decode()


def nv_sample_workspace_size(batch: int, vocab: int) -> int:
    return int(_native.load().nv_sample_workspace_size(batch, vocab))


def nv_sample(tokens: torch.Tensor, logits: torch.Tensor, temperatures: torch.Tensor,
              gumbel: torch.Tensor, workspace: Optional[torch.Tensor] = None,
              stream=None) -> None:
    """tokens: int32 [B] (device); logits: [B, V] float32 or bfloat16 (rows may be
    strided); temperatures: float32 [B]; gumbel: float32 [B, V] (rows may be strided).
    Without ``workspace`` the buffer cached for the device and stream is used."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [B, V] with contiguous rows")
    B, V = logits.shape
    if gumbel.shape != (B, V) or gumbel.stride(1) != 1 or gumbel.dtype != torch.float32:
        raise ValueError("gumbel must be float32 [B, V] with contiguous rows")
    if temperatures.dtype != torch.float32 or temperatures.numel() != B:
        raise ValueError("temperatures must be float32 with one entry per row")
    if tokens.dtype != torch.int32 or tokens.numel() != B:
        raise ValueError("tokens must be int32 with one entry per row")
    need = nv_sample_workspace_size(B, V)
    if workspace is None:
        workspace = decode_workspace(logits.device, need, stream)
    ws_ptr = 0 if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _native.load().nv_sample(
        _dev(tokens, "tokens"), _dev(logits, "logits", False), logits.stride(0),
        _dev(temperatures, "temperatures"), _dev(gumbel, "gumbel", False), gumbel.stride(0),
        B, V, _dtype_code(logits), ws_ptr, ws_bytes, _stream(stream, logits.device))
    _check("nv_sample", st)


def nv_paged_prefill_tile_rows(num_q_heads: int, num_kv_heads: int) -> int:
    return int(_native.load().nv_paged_prefill_tile_rows(num_q_heads, num_kv_heads))


# ---------------------------------------------------------------------------
# host metadata
# ---------------------------------------------------------------------------

def nv_prepare_decode(block_tables, context_lens, block_size: int, num_blocks: int,
                      with_schedule: bool = False):
    """Returns (slot_mapping, max_context_len) or, with_schedule, (slot_mapping,
    schedule, max_context_len); all host arrays."""
    bt = _i32(block_tables)
    cl = _i32(context_lens)
    batch = cl.shape[0]
    slots = np.empty(batch, dtype=np.int32)
    sched = np.empty(batch, dtype=np.int32) if with_schedule else None
    mx = ctypes.c_int32(0)
    st = _native.load().nv_prepare_decode(_ptr(bt), bt.shape[1] if bt.ndim == 2 else 1,
                                          _ptr(cl), batch, block_size, num_blocks,
                                          _ptr(slots), _ptr(sched) if with_schedule else None,
                                          ctypes.byref(mx))
    _check("nv_prepare_decode", st)
    if with_schedule:
        return slots, sched, int(mx.value)
    return slots, int(mx.value)


def nv_prepare_prefill(block_tables, num_cached, num_new, block_size: int, num_blocks: int,
                       pad_to: int = 1, tile_rows: int = 0):
    """Returns (cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, slot_mapping) and,
    with tile_rows > 0, also the [num_tiles, 2] tile schedule; all host arrays."""
    bt = _i32(block_tables)
    p = _i32(num_cached)
    n = _i32(num_new)
    S = n.shape[0]
    cap = int(-(-int(n.sum()) // pad_to) * pad_to) if S else 0
    cu_q = np.empty(S + 1, dtype=np.int32)
    cu_k = np.empty(S + 1, dtype=np.int32)
    slots = np.empty(max(cap, 1), dtype=np.int32)
    mq, mk, ns, nt = (ctypes.c_int32(0) for _ in range(4))
    tcap = int(sum(-(-int(x) // tile_rows) for x in n)) if tile_rows > 0 else 0
    tiles = np.empty((max(tcap, 1), 2), dtype=np.int32) if tile_rows > 0 else None
    st = _native.load().nv_prepare_prefill(
        _ptr(bt), bt.shape[1] if bt.ndim == 2 else 1, _ptr(p), _ptr(n), S, block_size,
        num_blocks, pad_to, _ptr(cu_q), _ptr(cu_k), ctypes.byref(mq), ctypes.byref(mk),
        _ptr(slots), cap, ctypes.byref(ns), tile_rows,
        _ptr(tiles) if tiles is not None else None, tcap, ctypes.byref(nt))
    _check("nv_prepare_prefill", st)
    res = (cu_q, cu_k, int(mq.value), int(mk.value), slots[:ns.value].copy())
    if tile_rows > 0:
        return res + (tiles[:nt.value].copy(),)
    return res
