"""Seeded generators for the five paged-attention workloads and for ad-hoc cases.

Value recipe: draw float32 N(0, 1) * sigma and, for bf16 workloads, round to
bfloat16 with round-to-nearest-even; the rounded bits are the canonical input
for every consumer.  bf16 tensors are held as raw ``uint16`` bit patterns,
fp32 tensors as ``float32``.

Structure recipe: physical blocks come from ``rng.permutation(num_blocks)``
popped in order (a toy free list); a block is never handed out twice except
the declared shared prefix blocks, which are full blocks referenced by several
sequences.  Block-table entries past a sequence's last block are -1.

The sequence of K/V rows each sequence holds is described *logically*: a
``Fill`` lists, per fill entry, a block-table row and a half-open range of
token positions whose rows must be in the pool before the timed/tested call,
plus the rows themselves packed in that order.  Shared prefix blocks are filled
exactly once, through a pseudo entry of their own.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

CONFIG_NAMES = ("C1", "C2", "C3", "C4", "C5")


# --------------------------------------------------------------------------
# dtype helpers (storage only)
# --------------------------------------------------------------------------

def np_storage_dtype(dtype: str):
    if dtype == "f32":
        return np.float32
    if dtype == "bf16":
        return np.uint16
    raise ValueError(dtype)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def poison_bits(dtype: str):
    """The quiet-NaN pattern used to fill every pool row that must never be read."""
    if dtype == "f32":
        return np.array([0x7FC00000], dtype=np.uint32).view(np.float32)[0]
    return np.uint16(0x7FC0)


def _draw(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "f32":
        return x
    return bf16_bits_from_f32(x)


def _nan_rows(n: int, hkv: int, d: int, dtype: str) -> np.ndarray:
    return np.full((n, hkv, d), poison_bits(dtype), dtype=np_storage_dtype(dtype))


# --------------------------------------------------------------------------
# data classes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    dtype: str            # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    sigma: float = 1.0

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


@dataclass
class Fill:
    """Rows that must be resident in the pool before the call under test."""
    block_tables: np.ndarray   # int32 [F, W], -1 padded
    start: np.ndarray          # int32 [F], first position to write
    end: np.ndarray            # int32 [F], one past the last position to write
    k: np.ndarray              # [sum(end - start), Hkv, D], packed in entry order
    v: np.ndarray

    @property
    def num_rows(self) -> int:
        return int(np.sum(self.end - self.start))


@dataclass
class DecodeStep:
    block_tables: np.ndarray   # int32 [B, W], -1 padded
    context_lens: np.ndarray   # int32 [B]; includes the token decoded this step
    q: np.ndarray              # [B, Hq, D]
    k_new: np.ndarray          # [B, Hkv, D]; row of the last position (L - 1)
    v_new: np.ndarray


@dataclass
class DecodeCase:
    name: str
    shape: Shape
    fill: Fill
    steps: List[DecodeStep]
    shared_blocks: List[int] = field(default_factory=list)

    @property
    def batch(self) -> int:
        return int(self.steps[0].context_lens.shape[0])


@dataclass
class PrefillCase:
    name: str
    shape: Shape
    fill: Fill                 # cached prefix rows (positions [0, num_cached))
    block_tables: np.ndarray   # int32 [S, W]
    num_cached: np.ndarray     # int32 [S]  (prefix tokens already in the pool)
    num_new: np.ndarray        # int32 [S]  (tokens computed this call)
    q: np.ndarray              # [sum(num_new), Hq, D]
    k_new: np.ndarray          # [n_pad, Hkv, D]; real rows first, then poisoned padding
    v_new: np.ndarray
    pad_to: int                # n_pad = roundup(sum(num_new), pad_to)
    causal: bool = True


# --------------------------------------------------------------------------
# toy free-list allocator
# --------------------------------------------------------------------------

class _FreeList:
    def __init__(self, rng: np.random.Generator, num_blocks: int):
        self._ids = [int(x) for x in rng.permutation(num_blocks)]
        self._next = 0

    def pop(self) -> int:
        if self._next >= len(self._ids):
            raise MemoryError("KV block pool exhausted")
        b = self._ids[self._next]
        self._next += 1
        return b

    @property
    def used(self) -> int:
        return self._next


def _blocks_for(length: int, block_size: int) -> int:
    return -(-length // block_size)


# --------------------------------------------------------------------------
# generic builders
# --------------------------------------------------------------------------

def build_decode(name: str, shape: Shape, lengths0: Sequence[int], *, seed: int,
                 steps: int = 1, num_sharers: int = 0, max_shared_blocks: int = 2,
                 share_unit: int = 1, table_width: Optional[int] = None) -> DecodeCase:
    """A decode workload of ``steps`` successive steps.

    Step t decodes one token per sequence with context length L0 + t; the token's
    own K/V row (position L0 + t - 1) is a new row.  When that position opens a
    new block, one block is popped from the free list.  ``num_sharers``
    sequences reference the same leading full blocks (1 .. ``max_shared_blocks``
    units of ``share_unit`` blocks, never the block the first write lands in).
    """
    ss = np.random.SeedSequence(seed)
    r_struct, r_kv, r_q = [np.random.default_rng(s) for s in ss.spawn(3)]
    bs, hkv, d, hq = shape.block_size, shape.num_kv_heads, shape.head_dim, shape.num_q_heads
    lengths0 = np.asarray(lengths0, dtype=np.int64)
    B = int(lengths0.shape[0])
    if np.any(lengths0 < 1):
        raise ValueError("decode context lengths include the decoded token and are >= 1")
    final_len = lengths0 + (steps - 1)
    W = table_width or max(1, int(max(_blocks_for(int(x), bs) for x in final_len))) if B else 1
    free = _FreeList(r_struct, shape.num_blocks)

    # shared prefix blocks (only full blocks strictly before the first written position)
    n_sh = np.zeros(B, dtype=np.int64)
    shared: List[int] = []
    if num_sharers:
        unit = bs * share_unit
        eligible = np.nonzero((lengths0 - 1) // unit >= 1)[0]
        if len(eligible) < num_sharers:
            raise ValueError("not enough sequences long enough to share a full block")
        sharers = np.sort(r_struct.choice(eligible, size=num_sharers, replace=False))
        want = r_struct.integers(1, max_shared_blocks, endpoint=True, size=num_sharers)
        n_sh[sharers] = np.minimum(want, (lengths0[sharers] - 1) // unit) * share_unit
        shared = [free.pop() for _ in range(int(n_sh.max()))]

    tables = np.full((B, W), -1, dtype=np.int32)
    nblk = np.zeros(B, dtype=np.int64)
    for b in range(B):
        for i in range(int(n_sh[b])):
            tables[b, i] = shared[i]
        nblk[b] = n_sh[b]
        while nblk[b] < _blocks_for(int(lengths0[b]), bs):
            tables[b, nblk[b]] = free.pop()
            nblk[b] += 1

    # logical rows: shared prefix rows are common to every sharer
    n_shared_rows = len(shared) * bs
    pre_k = _draw(r_kv, (n_shared_rows, hkv, d), shape.sigma, shape.dtype)
    pre_v = _draw(r_kv, (n_shared_rows, hkv, d), shape.sigma, shape.dtype)
    own_start = n_sh * bs
    total_own = int(np.sum(final_len - own_start))
    own_k = _draw(r_kv, (total_own, hkv, d), shape.sigma, shape.dtype)
    own_v = _draw(r_kv, (total_own, hkv, d), shape.sigma, shape.dtype)
    own_off = np.concatenate([[0], np.cumsum(final_len - own_start)])

    def own_row(arr, b, pos):
        return arr[own_off[b] + (pos - own_start[b])]

    # fill: shared pseudo entry first, then every sequence's private history
    f_tables, f_start, f_end, f_k, f_v = [], [], [], [], []
    if shared:
        row = np.full(W, -1, dtype=np.int32)
        row[:len(shared)] = shared
        f_tables.append(row)
        f_start.append(0)
        f_end.append(n_shared_rows)
        f_k.append(pre_k)
        f_v.append(pre_v)
    for b in range(B):
        s0, e0 = int(own_start[b]), int(lengths0[b] - 1)
        f_tables.append(tables[b].copy())
        f_start.append(s0)
        f_end.append(max(s0, e0))
        lo = own_off[b]
        f_k.append(own_k[lo:lo + max(0, e0 - s0)])
        f_v.append(own_v[lo:lo + max(0, e0 - s0)])
    sd = np_storage_dtype(shape.dtype)
    fill = Fill(
        block_tables=np.array(f_tables, dtype=np.int32).reshape(-1, W),
        start=np.array(f_start, dtype=np.int32), end=np.array(f_end, dtype=np.int32),
        k=np.concatenate(f_k) if f_k else np.zeros((0, hkv, d), sd),
        v=np.concatenate(f_v) if f_v else np.zeros((0, hkv, d), sd))

    out_steps: List[DecodeStep] = []
    for t in range(steps):
        L = lengths0 + t
        for b in range(B):
            while nblk[b] < _blocks_for(int(L[b]), bs):
                tables[b, nblk[b]] = free.pop()
                nblk[b] += 1
        q = _draw(r_q, (B, hq, d), shape.sigma, shape.dtype)
        kn = np.stack([own_row(own_k, b, int(L[b] - 1)) for b in range(B)]) if B else np.zeros((0, hkv, d), sd)
        vn = np.stack([own_row(own_v, b, int(L[b] - 1)) for b in range(B)]) if B else np.zeros((0, hkv, d), sd)
        out_steps.append(DecodeStep(block_tables=tables.copy(), context_lens=L.astype(np.int32),
                                    q=q, k_new=kn, v_new=vn))
    return DecodeCase(name=name, shape=shape, fill=fill, steps=out_steps, shared_blocks=shared)


def build_prefill(name: str, shape: Shape, num_new: Sequence[int], num_cached: Sequence[int], *,
                  seed: int, pad_to: int = 128, causal: bool = True,
                  table_width: Optional[int] = None) -> PrefillCase:
    """A packed varlen prefill: sequence s has ``num_cached[s]`` prefix rows already in the
    pool (private blocks) and ``num_new[s]`` new tokens whose K/V are stored this call."""
    ss = np.random.SeedSequence(seed)
    r_struct, r_kv, r_q = [np.random.default_rng(s) for s in ss.spawn(3)]
    bs, hkv, d, hq = shape.block_size, shape.num_kv_heads, shape.head_dim, shape.num_q_heads
    n = np.asarray(num_new, dtype=np.int64)
    p = np.asarray(num_cached, dtype=np.int64)
    S = int(n.shape[0])
    total = n + p
    W = table_width or max(1, int(max((_blocks_for(int(x), bs) for x in total), default=1)))
    free = _FreeList(r_struct, shape.num_blocks)
    tables = np.full((S, W), -1, dtype=np.int32)
    for s in range(S):
        for i in range(_blocks_for(int(total[s]), bs)):
            tables[s, i] = free.pop()
    pk = _draw(r_kv, (int(p.sum()), hkv, d), shape.sigma, shape.dtype)
    pv = _draw(r_kv, (int(p.sum()), hkv, d), shape.sigma, shape.dtype)
    nk = _draw(r_kv, (int(n.sum()), hkv, d), shape.sigma, shape.dtype)
    nv = _draw(r_kv, (int(n.sum()), hkv, d), shape.sigma, shape.dtype)
    q = _draw(r_q, (int(n.sum()), hq, d), shape.sigma, shape.dtype)
    n_real = int(n.sum())
    n_pad = -(-n_real // pad_to) * pad_to if pad_to > 1 else n_real
    pad = _nan_rows(n_pad - n_real, hkv, d, shape.dtype)
    fill = Fill(block_tables=tables.copy(), start=np.zeros(S, np.int32), end=p.astype(np.int32),
                k=pk, v=pv)
    return PrefillCase(name=name, shape=shape, fill=fill, block_tables=tables,
                       num_cached=p.astype(np.int32), num_new=n.astype(np.int32), q=q,
                       k_new=np.concatenate([nk, pad]), v_new=np.concatenate([nv, pad]),
                       pad_to=pad_to, causal=causal)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------

SHAPES = {
    "C1": Shape("f32", 2, 1, 64, 16, 64, 1.0),
    "C2": Shape("bf16", 16, 8, 128, 256, 2048, 0.5),
    "C3": Shape("bf16", 16, 8, 128, 256, 2048, 0.5),
    "C4": Shape("bf16", 32, 8, 128, 256, 1536, 1.0),
    "C5": Shape("bf16", 32, 8, 128, 256, 2048, 0.5),
}


def decode_config(name: str, *, batch: Optional[int] = None, steps: Optional[int] = None,
                  num_blocks: Optional[int] = None, seed: Optional[int] = None,
                  block_size: Optional[int] = None, tp: int = 1) -> DecodeCase:
    """C1-C4.  ``batch``/``steps``/``num_blocks`` shrink a workload for CPU-sized tests
    (same recipe, smaller draw); the defaults are the full workloads.

    ``block_size`` redraws the workload with another block size: the same lengths and
    pool bytes (``num_blocks`` scaled by the size ratio unless given), and C3's shared
    prefixes cover the same 1-2 x 256 tokens (as whole blocks of the new size).

    ``tp`` gives one GPU's share of the workload under head-parallel sharding over ``tp``
    GPUs: num_q_heads / tp query heads and num_kv_heads / tp KV heads, the same lengths,
    block tables and sharing (each GPU holds its heads' slice of every block)."""
    idx = CONFIG_NAMES.index(name)
    sh = SHAPES[name]
    if tp < 1 or sh.num_kv_heads % tp:
        raise ValueError(f"{name} has {sh.num_kv_heads} KV heads: cannot shard over {tp}")
    if tp > 1:
        sh = Shape(sh.dtype, sh.num_q_heads // tp, sh.num_kv_heads // tp, sh.head_dim,
                   sh.block_size, sh.num_blocks, sh.sigma)
    bs = sh.block_size if block_size is None else int(block_size)
    if bs < 1 or (sh.block_size * sh.num_blocks) % bs:
        raise ValueError(f"block size {bs} does not divide the {name} pool")
    nb = num_blocks if num_blocks is not None else sh.block_size * sh.num_blocks // bs
    sh = Shape(sh.dtype, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, bs, nb, sh.sigma)
    seed = 1000 + idx if seed is None else seed
    len_rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    if name == "C1":
        lengths = [1, 17, 64, 200]
        return build_decode(name, sh, lengths, seed=seed, steps=steps or 1)
    if name == "C2":
        B = batch or 64
        lengths = len_rng.integers(128, 4096, endpoint=True, size=B)
        return build_decode(name, sh, lengths, seed=seed, steps=steps or 1)
    if name == "C3":
        B = batch or 256
        lengths = len_rng.integers(100, 1024, endpoint=True, size=B)
        n_share = int(round(0.3 * B))
        return build_decode(name, sh, lengths, seed=seed, steps=steps or 50,
                            num_sharers=n_share, max_shared_blocks=2,
                            share_unit=max(1, 256 // bs))
    if name == "C4":
        B = batch or 8
        return build_decode(name, sh, [32768] * B, seed=seed, steps=steps or 1)
    raise ValueError(f"{name} is not a decode workload")


def prefill_config(name: str = "C5", *, num_seqs: Optional[int] = None,
                   max_new: int = 1024, seed: Optional[int] = None,
                   block_size: Optional[int] = None) -> PrefillCase:
    """C5.  ``block_size`` redraws it with another block size: the same lengths, prefixes
    of 0-4 x 256 tokens and pool bytes."""
    if name != "C5":
        raise ValueError(f"{name} is not a prefill workload")
    sh = SHAPES[name]
    if block_size is not None:
        bs = int(block_size)
        if bs < 1 or 256 % bs or (sh.block_size * sh.num_blocks) % bs:
            raise ValueError(f"block size {bs} does not divide the C5 prefixes")
        sh = Shape(sh.dtype, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, bs,
                   sh.block_size * sh.num_blocks // bs, sh.sigma)
    seed = 1000 + CONFIG_NAMES.index(name) if seed is None else seed
    S = num_seqs or 16
    len_rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    n = len_rng.integers(min(100, max_new), max_new, endpoint=True, size=S)
    p = 256 * len_rng.integers(0, 4, endpoint=True, size=S)
    return build_prefill(name, sh, n, p, seed=seed, pad_to=128, causal=True)


# --------------------------------------------------------------------------
# token sampler workload
# --------------------------------------------------------------------------

@dataclass
class SamplerCase:
    """Logits of one decode step, per-row temperatures and the Gumbel noise the
    sampler consumes.  ``logits`` is float32 or raw bfloat16 bits (uint16)."""
    dtype: str
    logits: np.ndarray        # [batch, vocab]
    temperatures: np.ndarray  # float32 [batch]; 0 = greedy row
    gumbel: np.ndarray        # float32 [batch, vocab], standard Gumbel draws

    @property
    def batch(self) -> int:
        return int(self.logits.shape[0])

    @property
    def vocab(self) -> int:
        return int(self.logits.shape[1])


def sampler_case(batch: int = 256, vocab: int = 151936, *, dtype: str = "bf16",
                 sigma: float = 2.0, greedy_fraction: float = 0.125,
                 t_range=(0.5, 1.0), seed: int = 2000) -> SamplerCase:
    """Seeded sampler input.  Defaults: the decode batch of 256 over a Qwen3-sized
    vocabulary of 151,936 entries; logits N(0, 1) * 2 (rounded to bf16 for bf16);
    round(batch / 8) rows (seeded choice) at temperature 0, the others U[0.5, 1.0);
    noise from numpy's Gumbel(0, 1) generator, stored as float32."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, batch, vocab]))
    logits = _draw(rng, (batch, vocab), sigma, dtype)
    temps = rng.uniform(t_range[0], t_range[1], size=batch).astype(np.float32)
    n_greedy = int(round(batch * greedy_fraction))
    if n_greedy:
        temps[rng.choice(batch, size=n_greedy, replace=False)] = 0.0
    gumbel = np.empty((batch, vocab), dtype=np.float32)
    for b in range(batch):                       # row by row: bounded float64 temporaries
        gumbel[b] = rng.gumbel(size=vocab)
    return SamplerCase(dtype, logits, temps, gumbel)
