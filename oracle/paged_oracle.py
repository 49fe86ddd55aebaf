"""Plain float64 reference for the paged KV-cache attention path (test infrastructure).

Layouts (the method's own terms):
  k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim], native dtype
  block_tables     : int [num_seqs, width]; row s lists the physical block of each
                     logical block of sequence s, unused tail entries are -1
  slot_mapping     : int [n]; one-dimensional physical row index per new token, -1 = skip
  q / out          : [tokens, num_q_heads, head_dim]

Inputs arrive in their storage form: float32 arrays, or raw bfloat16 bit patterns
held as uint16.  Every arithmetic step below runs in float64 on the exact values
those bits encode.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


# ---------------------------------------------------------------------------
# numbers
# ---------------------------------------------------------------------------

def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a float32 array or of raw bfloat16 bits (uint16).

    A bfloat16 is the upper half of an IEEE binary32 word, so widening the bits
    by 16 zero bits gives the binary32 with the same value.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype}")


def new_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
             storage_dtype, fill) -> np.ndarray:
    """A physical K or V pool: one pre-allocated array split into fixed-size blocks
    (nano-vllm walkthrough, section 六: the runner pre-allocates the cache)."""
    return np.full((num_blocks, block_size, num_kv_heads, head_dim), fill, dtype=storage_dtype)


# ---------------------------------------------------------------------------
# metadata: logical position -> physical slot
# ---------------------------------------------------------------------------

def slot_of(block_table_row: np.ndarray, pos: int, block_size: int) -> int:
    """Physical slot of logical token ``pos`` of one sequence.

    The paging article (section 4.1) locates token t in logical block t // B at
    offset t % B; the walkthrough (section 八) names the one-dimensional index of
    that physical row the slot.  With the pool viewed as [num_blocks * B, ...]
    the physical block id b and offset o give row b * B + o.
    """
    logical_block = pos // block_size
    offset = pos % block_size
    physical_block = int(block_table_row[logical_block])
    if physical_block < 0:
        raise IndexError("position maps to an unassigned block-table entry")
    return physical_block * block_size + offset


def decode_slot_mapping(block_tables: np.ndarray, context_lens: np.ndarray,
                        block_size: int) -> Tuple[np.ndarray, int]:
    """Decode metadata (walkthrough, section 七: prepare_decode passes each sequence's
    current length and the slot of its last token).  The token decoded this step is
    at position L - 1 and its K/V row is stored there."""
    slots = np.empty(len(context_lens), dtype=np.int32)
    for b, L in enumerate(context_lens):
        slots[b] = slot_of(block_tables[b], int(L) - 1, block_size)
    max_len = int(max(context_lens)) if len(context_lens) else 0
    return slots, max_len


def prefill_metadata(block_tables: np.ndarray, num_cached: np.ndarray, num_new: np.ndarray,
                     block_size: int, pad_to: int):
    """Prefill metadata (walkthrough, section 七: prepare_prefill builds cu_seqlens_q/k,
    max_seqlen_q/k and the slot of every newly written token).

    Sequence s computes ``num_new[s]`` tokens at positions num_cached[s] .. num_cached[s]
    + num_new[s] - 1 and attends over all num_cached[s] + num_new[s] keys.  The slot list
    covers the new tokens in packed order; rows appended to reach a multiple of
    ``pad_to`` get slot -1.
    """
    S = len(num_new)
    cu_q = np.zeros(S + 1, dtype=np.int32)
    cu_k = np.zeros(S + 1, dtype=np.int32)
    slots = []
    for s in range(S):
        p, n = int(num_cached[s]), int(num_new[s])
        cu_q[s + 1] = cu_q[s] + n
        cu_k[s + 1] = cu_k[s] + p + n
        for t in range(p, p + n):
            slots.append(slot_of(block_tables[s], t, block_size))
    n_real = len(slots)
    n_pad = -(-n_real // pad_to) * pad_to if pad_to > 1 else n_real
    slots.extend([-1] * (n_pad - n_real))
    max_q = int(max(num_new)) if S else 0
    max_k = int(max(np.asarray(num_new) + np.asarray(num_cached))) if S else 0
    return cu_q, cu_k, max_q, max_k, np.array(slots, dtype=np.int32)


def fill_slot_mapping(block_tables: np.ndarray, start: np.ndarray, end: np.ndarray,
                      block_size: int) -> np.ndarray:
    """Slots of positions [start[i], end[i]) of each entry, packed in entry order."""
    out = []
    for i in range(len(start)):
        for t in range(int(start[i]), int(end[i])):
            out.append(slot_of(block_tables[i], t, block_size))
    return np.array(out, dtype=np.int32)


# ---------------------------------------------------------------------------
# store_kvcache
# ---------------------------------------------------------------------------

def store_kvcache(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
                  slot_mapping: np.ndarray) -> None:
    """Write row i of k / v into the pool row named by slot_mapping[i], in place.

    Walkthrough section 七: before attention a lightweight kernel puts this step's K/V
    into the pre-allocated cache by slot_mapping; gitcode summary section 三.4 calls it a
    plain copy.  A slot of -1 leaves the pool untouched.  Values are copied in their
    storage dtype (bit for bit).
    """
    block_size = k_cache.shape[1]
    for i, s in enumerate(np.asarray(slot_mapping)):
        s = int(s)
        if s == -1:
            continue
        blk, off = divmod(s, block_size)
        k_cache[blk, off] = k[i]
        v_cache[blk, off] = v[i]


# ---------------------------------------------------------------------------
# gather + attention
# ---------------------------------------------------------------------------

def gather(cache: np.ndarray, block_table_row: np.ndarray, length: int) -> np.ndarray:
    """Logical rows 0 .. length-1 of one sequence, gathered from its blocks
    (paging article, sections 4.1 and 5.3: gather the scattered blocks into contiguous
    K/V, then run ordinary attention).  Returns float64 [length, Hkv, D]."""
    block_size = cache.shape[1]
    rows = [cache[int(block_table_row[t // block_size]), t % block_size] for t in range(length)]
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=np.float64)
    return to_f64(np.stack(rows))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           last_key: np.ndarray) -> np.ndarray:
    """softmax(q K^T * scale) V for each query row (deep dive, section 1.2), where query
    row i sees keys 0 .. last_key[i] only.  q: [n, D], K, V: [Lk, D]; float64."""
    s = (q @ K.T) * scale
    keys = np.arange(K.shape[0])[None, :]
    s = np.where(keys <= np.asarray(last_key)[:, None], s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ V) / np.sum(p, axis=1, keepdims=True)


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float) -> np.ndarray:
    """One query token per sequence attends all ``context_lens[b]`` keys of its sequence
    (walkthrough section 七: the decode call takes the cache, cache_seqlens=context_lens and
    the block table).  GQA: query head h reads KV head h // (Hq / Hkv) (deep dive,
    section 3.2.1: each group of query heads shares one K/V pair; the K/V heads are
    repeated num_kv_groups times in order).  Returns float64 [B, Hq, D]."""
    q64 = to_f64(q)
    B, Hq, D = q64.shape
    Hkv = k_cache.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K = gather(k_cache, block_tables[b], L)
        V = gather(v_cache, block_tables[b], L)
        for h in range(Hq):
            j = h // g
            out[b, h] = attend(q64[b, h][None, :], K[:, j], V[:, j], scale,
                               np.array([L - 1]))[0]
    return out


def paged_prefill(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables,
                  scale: float, causal: bool = True) -> np.ndarray:
    """Packed varlen prefill (walkthrough section 七: the prefill call takes q, the cache,
    cu_seqlens_q/k, max_seqlen_q/k, causal=True and the block table).

    Sequence s has n = cu_q[s+1] - cu_q[s] query rows and k = cu_k[s+1] - cu_k[s] keys,
    all read from the pool through its block table.  Only the uncached tail is computed,
    so query row i is the token at absolute position (k - n) + i; under the causal mask it
    sees keys 0 .. (k - n) + i.  Without the mask it sees all k keys.  Returns float64
    [cu_q[-1], Hq, D]."""
    q64 = to_f64(q)
    Nq, Hq, D = q64.shape
    Hkv = k_cache.shape[2]
    g = Hq // Hkv
    out = np.zeros((Nq, Hq, D), dtype=np.float64)
    for s in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        n = q1 - q0
        k = int(cu_seqlens_k[s + 1]) - int(cu_seqlens_k[s])
        if n == 0:
            continue
        K = gather(k_cache, block_tables[s], k)
        V = gather(v_cache, block_tables[s], k)
        if causal:
            last = (k - n) + np.arange(n)
        else:
            last = np.full(n, k - 1)
        for h in range(Hq):
            j = h // g
            out[q0:q1, h] = attend(q64[q0:q1, h], K[:, j], V[:, j], scale, last)
    return out
