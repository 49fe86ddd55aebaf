"""Plain reference of the KV block manager (test infrastructure, not product code).

Follows the nano-vllm walkthrough (xingyun3d.csdn.net), section 五 "KV Block 管理":
a pool of fixed-size blocks, each with a block id, a reference count, a content hash
and its token ids; a hash -> block id index for prefix reuse; a free pool and a used
set.  allocate walks a prompt block by block with a rolling hash (a hit raises the
block's count and adds a block of cached tokens, a miss takes a block from the free
pool); may_append opens a block when a decoded token is the first of a new block and
seals a block's hash once it is full; deallocate lowers every count of a sequence and
returns blocks that reach zero.  Only full blocks are hashed and shared.  Section 八
of the same article gives the slot of a token: block_table[p // block_size] *
block_size + p % block_size.

Where the article leaves a step open this file takes these readings:
  * hash: XXH64 (seed 0) of the previous block's hash as 8 little-endian bytes (absent
    for the first block) followed by the block's token ids as int32 little-endian; the
    library routine xxhash.xxh64_intdigest computes it;
  * a hit also requires the block's stored token ids to equal the new block's;
  * once a block misses, every later block of the prompt misses (cached tokens form a
    prefix);
  * the block holding the prompt's last token never hits, so a prefill always has at
    least one token to compute and never writes into a shared block;
  * the free pool is first-in first-out: blocks are taken from its front (initially
    0, 1, 2, ...) and released to its back; a freed block keeps its hash and tokens
    until it is taken again, and a later hit on it takes it back out of the pool;
  * a newly hashed block becomes the index entry for its hash (latest wins);
  * deallocate releases a sequence's blocks from its last to its first;
  * can_allocate asks for as many free blocks as the prompt has blocks, hits ignored;
    can_append asks for one when the next token starts a new block.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence as Seq

import numpy as np
import xxhash


def compute_hash(token_ids: Seq[int], prefix: Optional[int]) -> int:
    """Rolling block hash: XXH64 over (previous hash, this block's token ids)."""
    data = b"" if prefix is None else int(prefix).to_bytes(8, "little")
    data += np.asarray(token_ids, dtype="<i4").tobytes()
    return xxhash.xxh64_intdigest(data, seed=0)


class Block:
    def __init__(self, block_id: int):
        self.block_id = block_id
        self.ref_count = 0
        self.hash: Optional[int] = None
        self.token_ids: List[int] = []


class Sequence:
    def __init__(self, seq_id: int, token_ids: Seq[int]):
        self.seq_id = seq_id
        self.token_ids = [int(t) for t in token_ids]
        self.block_table: List[int] = []
        self.num_cached_tokens = 0


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.block_size = block_size
        self.blocks = [Block(i) for i in range(num_blocks)]
        self.hash_to_block_id: Dict[int, int] = {}
        self.free_block_ids: List[int] = list(range(num_blocks))
        self.used_block_ids = set()
        self.seqs: Dict[int, Sequence] = {}

    # -- helpers -------------------------------------------------------------
    def _num_blocks(self, n_tokens: int) -> int:
        return -(-n_tokens // self.block_size)

    def _take(self, block_id: int) -> Block:
        """Move a block from the free pool to the used set with one reference."""
        self.free_block_ids.remove(block_id)
        self.used_block_ids.add(block_id)
        blk = self.blocks[block_id]
        blk.ref_count = 1
        return blk

    def _take_fresh(self) -> Block:
        """A miss: the block at the front of the free pool, its old content dropped."""
        blk = self._take(self.free_block_ids[0])
        if blk.hash is not None and self.hash_to_block_id.get(blk.hash) == blk.block_id:
            del self.hash_to_block_id[blk.hash]
        blk.hash = None
        blk.token_ids = []
        return blk

    def _seal(self, blk: Block, token_ids: Seq[int], prefix: Optional[int]):
        blk.hash = compute_hash(token_ids, prefix)
        blk.token_ids = list(token_ids)
        self.hash_to_block_id[blk.hash] = blk.block_id

    # -- the article's operations ----------------------------------------------
    def can_allocate(self, n_tokens: int) -> bool:
        return len(self.free_block_ids) >= self._num_blocks(n_tokens)

    def allocate(self, seq_id: int, token_ids: Seq[int]) -> int:
        """Prefill: build the block table of a new sequence; returns its cached tokens."""
        if seq_id in self.seqs or len(token_ids) < 1:
            raise ValueError("allocate needs a new sequence id and a non-empty prompt")
        if not self.can_allocate(len(token_ids)):
            raise MemoryError("not enough free blocks")
        seq = Sequence(seq_id, token_ids)
        bs, n = self.block_size, len(seq.token_ids)
        nblk = self._num_blocks(n)
        prefix: Optional[int] = None
        missed = False
        for i in range(nblk):
            toks = seq.token_ids[i * bs:(i + 1) * bs]
            full = len(toks) == bs
            h = compute_hash(toks, prefix) if full else None
            hit_id = None
            if full and i < nblk - 1 and not missed:
                cand = self.hash_to_block_id.get(h)
                if cand is not None and self.blocks[cand].token_ids == toks:
                    hit_id = cand
            if hit_id is not None:
                seq.num_cached_tokens += bs
                if hit_id in self.used_block_ids:
                    self.blocks[hit_id].ref_count += 1
                else:
                    self._take(hit_id)
                seq.block_table.append(hit_id)
            else:
                missed = True
                blk = self._take_fresh()
                if full:
                    self._seal(blk, toks, prefix)
                seq.block_table.append(blk.block_id)
            prefix = h
        self.seqs[seq_id] = seq
        return seq.num_cached_tokens

    def can_append(self, seq_id: int) -> bool:
        n_next = len(self.seqs[seq_id].token_ids) + 1
        need = 1 if (n_next - 1) % self.block_size == 0 else 0
        return len(self.free_block_ids) >= need

    def append_token(self, seq_id: int, token_id: int):
        """Decode: the sequence grows by one token; may_append then fixes its blocks."""
        if not self.can_append(seq_id):
            raise MemoryError("not enough free blocks")
        seq = self.seqs[seq_id]
        seq.token_ids.append(int(token_id))
        self.may_append(seq)

    def may_append(self, seq: Sequence):
        bs, n = self.block_size, len(seq.token_ids)
        if (n - 1) % bs == 0:          # the token opens a new block
            seq.block_table.append(self._take_fresh().block_id)
        if n % bs == 0:                # the last block is now full: seal its hash
            last = self.blocks[seq.block_table[-1]]
            prefix = self.blocks[seq.block_table[-2]].hash if len(seq.block_table) > 1 else None
            self._seal(last, seq.token_ids[n - bs:n], prefix)

    def deallocate(self, seq_id: int):
        seq = self.seqs.pop(seq_id)
        for block_id in reversed(seq.block_table):
            blk = self.blocks[block_id]
            blk.ref_count -= 1
            if blk.ref_count == 0:
                self.used_block_ids.discard(block_id)
                self.free_block_ids.append(block_id)

    # -- kernel metadata -------------------------------------------------------
    def slot(self, seq_id: int, position: int) -> int:
        seq = self.seqs[seq_id]
        return seq.block_table[position // self.block_size] * self.block_size + \
            position % self.block_size

    def decode_step(self, seq_ids: Seq[int], new_tokens: Seq[int], width: int):
        """Append one token to each sequence; return (block_tables [B, width] padded with
        -1, context_lens [B], slot_mapping [B]) for the decode of those tokens."""
        if len(set(seq_ids)) != len(seq_ids):
            raise ValueError("duplicate sequence in a decode batch")
        need = sum(1 for s in seq_ids if len(self.seqs[s].token_ids) % self.block_size == 0)
        if need > len(self.free_block_ids):
            raise MemoryError("not enough free blocks")
        if any(self._num_blocks(len(self.seqs[s].token_ids) + 1) > width for s in seq_ids):
            raise ValueError("block table width too small")
        B = len(seq_ids)
        tables = np.full((B, width), -1, dtype=np.int32)
        lens = np.zeros(B, dtype=np.int32)
        slots = np.zeros(B, dtype=np.int32)
        for b, (s, tok) in enumerate(zip(seq_ids, new_tokens)):
            self.append_token(s, tok)
            seq = self.seqs[s]
            tables[b, :len(seq.block_table)] = seq.block_table
            lens[b] = len(seq.token_ids)
            slots[b] = self.slot(s, lens[b] - 1)
        return tables, lens, slots

    def prefill_step(self, seq_ids: Seq[int], prompts: Seq[Seq[int]], width: int):
        """Allocate each new sequence; return (block_tables [S, width] padded with -1,
        num_cached [S])."""
        if len(set(seq_ids)) != len(seq_ids) or any(s in self.seqs for s in seq_ids):
            raise ValueError("prefill needs distinct new sequence ids")
        if any(len(p) < 1 for p in prompts):
            raise ValueError("empty prompt")
        if sum(self._num_blocks(len(p)) for p in prompts) > len(self.free_block_ids):
            raise MemoryError("not enough free blocks")
        if any(self._num_blocks(len(p)) > width for p in prompts):
            raise ValueError("block table width too small")
        S = len(seq_ids)
        tables = np.full((S, width), -1, dtype=np.int32)
        cached = np.zeros(S, dtype=np.int32)
        for i, (s, p) in enumerate(zip(seq_ids, prompts)):
            cached[i] = self.allocate(s, p)
            bt = self.seqs[s].block_table
            tables[i, :len(bt)] = bt
        return tables, cached
