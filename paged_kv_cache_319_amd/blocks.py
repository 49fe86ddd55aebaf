"""Python face of the host-side KV block manager (include/nvpaged_blocks.h).

Marshalling only: every operation runs in libnvpaged.so's C++ manager; this class
holds its handle and converts numpy arrays to int32/int64 buffers.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import _native
from .api import NvError

NV_OK = 0


def _check(fn: str, status: int):
    if status != NV_OK:
        raise NvError(fn, status)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_native.c_i32p)


def _p64(a: np.ndarray):
    return a.ctypes.data_as(_native.c_i64p)


def nv_bm_xxh64(data: bytes, seed: int = 0) -> int:
    buf = ctypes.create_string_buffer(bytes(data), max(1, len(data)))
    return int(_native.load().nv_bm_xxh64(buf, len(data), seed))


class BlockManager:
    """Handle to a C++ block manager of num_blocks blocks of block_size tokens."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _native.load()
        h = ctypes.c_void_p()
        _check("nv_bm_create", self._lib.nv_bm_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if getattr(self, "_h", None):
            self._lib.nv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # -- the manager's operations ----------------------------------------------------
    @property
    def num_free_blocks(self) -> int:
        return int(self._lib.nv_bm_num_free_blocks(self._h))

    def can_allocate(self, num_tokens: int) -> bool:
        ok = ctypes.c_int32()
        _check("nv_bm_can_allocate", self._lib.nv_bm_can_allocate(self._h, num_tokens,
                                                                  ctypes.byref(ok)))
        return bool(ok.value)

    def allocate(self, seq_id: int, token_ids) -> int:
        t = _i32(token_ids)
        cached = ctypes.c_int32()
        _check("nv_bm_allocate", self._lib.nv_bm_allocate(self._h, seq_id, _p32(t), len(t),
                                                          ctypes.byref(cached)))
        return int(cached.value)

    def can_append(self, seq_id: int) -> bool:
        ok = ctypes.c_int32()
        _check("nv_bm_can_append", self._lib.nv_bm_can_append(self._h, seq_id, ctypes.byref(ok)))
        return bool(ok.value)

    def append_token(self, seq_id: int, token_id: int):
        _check("nv_bm_append_token", self._lib.nv_bm_append_token(self._h, seq_id, token_id))

    def deallocate(self, seq_id: int):
        _check("nv_bm_deallocate", self._lib.nv_bm_deallocate(self._h, seq_id))

    # -- inspection --------------------------------------------------------------------
    def sequence(self, seq_id: int) -> Tuple[int, int, List[int]]:
        """(num_tokens, num_cached_tokens, block table) of a live sequence."""
        n, c, nb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("nv_bm_get_sequence", self._lib.nv_bm_get_sequence(
            self._h, seq_id, ctypes.byref(n), ctypes.byref(c), None, 0, ctypes.byref(nb)))
        table = np.zeros(max(1, nb.value), dtype=np.int32)
        _check("nv_bm_get_sequence", self._lib.nv_bm_get_sequence(
            self._h, seq_id, None, None, _p32(table), len(table), ctypes.byref(nb)))
        return int(n.value), int(c.value), table[:nb.value].tolist()

    def block(self, block_id: int) -> Tuple[int, Optional[int]]:
        """(reference count, hash or None) of a block."""
        ref, has, h = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_uint64()
        _check("nv_bm_get_block", self._lib.nv_bm_get_block(
            self._h, block_id, ctypes.byref(ref), ctypes.byref(has), ctypes.byref(h)))
        return int(ref.value), (int(h.value) if has.value else None)

    def free_blocks(self) -> List[int]:
        n = ctypes.c_int32()
        _check("nv_bm_get_free_blocks", self._lib.nv_bm_get_free_blocks(
            self._h, None, 0, ctypes.byref(n)))
        ids = np.zeros(max(1, n.value), dtype=np.int32)
        _check("nv_bm_get_free_blocks", self._lib.nv_bm_get_free_blocks(
            self._h, _p32(ids), len(ids), ctypes.byref(n)))
        return ids[:n.value].tolist()

    # -- step metadata -----------------------------------------------------------------
    def decode_step(self, seq_ids: Sequence[int], new_tokens, width: int):
        """Append one token per sequence; returns (block_tables [B, width],
        context_lens [B], slot_mapping [B]) as int32 numpy arrays."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        toks = _i32(new_tokens)
        B = len(ids)
        if len(toks) != B:
            raise ValueError("one new token per sequence")
        tables = np.zeros((B, width), dtype=np.int32)
        lens = np.zeros(B, dtype=np.int32)
        slots = np.zeros(B, dtype=np.int32)
        _check("nv_bm_decode_step", self._lib.nv_bm_decode_step(
            self._h, _p64(ids), _p32(toks), B, _p32(tables), width, _p32(lens), _p32(slots)))
        return tables, lens, slots

    def prefill_step(self, seq_ids: Sequence[int], prompts: Sequence[Sequence[int]], width: int):
        """Allocate new sequences; returns (block_tables [S, width], num_cached [S])."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        S = len(ids)
        if len(prompts) != S:
            raise ValueError("one prompt per sequence")
        cu = _i32(np.concatenate([[0], np.cumsum([len(p) for p in prompts])]))
        toks = _i32(np.concatenate([np.asarray(p, dtype=np.int64) for p in prompts])
                    if S else np.zeros(0))
        if len(toks) == 0:
            toks = np.zeros(1, dtype=np.int32)
        tables = np.zeros((max(S, 1), width), dtype=np.int32)
        cached = np.zeros(max(S, 1), dtype=np.int32)
        _check("nv_bm_prefill_step", self._lib.nv_bm_prefill_step(
            self._h, _p64(ids), _p32(cu), _p32(toks), S, _p32(tables), width, _p32(cached)))
        return tables[:S], cached[:S]
