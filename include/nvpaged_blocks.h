/*
 * nvpaged — host-side KV block manager.
 *
 * The nano-vllm walkthrough (xingyun3d.csdn.net), section 五 "KV Block 管理":
 * a pool of num_blocks fixed-size blocks, each with a block id, a reference
 * count, a content hash and its token ids; an index from hash to block id for
 * prefix reuse; a free pool and a used set.  allocate walks a prompt block by
 * block with a rolling hash: a hit raises the block's count and adds a block of
 * cached tokens, a miss takes a block from the free pool.  In decode a block is
 * opened when a token is the first of a new block and its hash is sealed once it
 * is full; deallocate lowers every count of a sequence and returns blocks that
 * reach zero.  The manager hands out block ids only; the K/V cache itself is
 * the caller's [num_blocks, block_size, num_kv_heads, head_dim] device array,
 * addressed through block tables and slot mappings (section 八).
 *
 * Rules where the article leaves a step open:
 *   - only full blocks are hashed and shared; the hash of block i is XXH64
 *     (seed 0) of block i-1's hash as 8 little-endian bytes (nothing for i = 0)
 *     followed by block i's token ids as little-endian int32;
 *   - a hit needs the indexed block's token ids to equal the prompt block's;
 *     after the first miss every later block of the prompt misses, so cached
 *     tokens are a prefix; the block holding the prompt's last token never hits,
 *     so a prefill always computes at least one token and never writes into a
 *     shared block;
 *   - the free pool is first-in first-out (initially 0, 1, 2, ...); a released
 *     block keeps its hash and tokens until it is taken again, and a hit on it
 *     takes it back out of the pool; a newly hashed block becomes the index
 *     entry for its hash; deallocate releases a sequence's blocks last to first;
 *   - can_allocate asks for as many free blocks as the prompt has blocks.
 *
 * Ownership and threading: nv_bm_create allocates the manager's host state and
 * nv_bm_destroy frees it; nothing here touches the GPU.  A handle must not be
 * used from two threads at once.  Every pointer argument is caller-owned host
 * memory.  Errors: NV_ERR_INVALID_ARG for null pointers, bad sizes, unknown or
 * duplicate sequence ids and block tables too narrow; NV_ERR_OUT_OF_BLOCKS when
 * the free pool is too small.  A call that returns an error changes nothing.
 */
#ifndef NVPAGED_BLOCKS_H
#define NVPAGED_BLOCKS_H

#include <stdint.h>

#include "nvpaged.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nv_block_manager nv_block_manager;

/* A pool of num_blocks blocks of block_size tokens (both >= 1), all free. */
nv_status nv_bm_create(int32_t num_blocks, int32_t block_size, nv_block_manager** out);
void nv_bm_destroy(nv_block_manager* bm);

int32_t nv_bm_num_free_blocks(const nv_block_manager* bm);

/* *ok = 1 if a prompt of num_tokens tokens can be allocated now, else 0. */
nv_status nv_bm_can_allocate(const nv_block_manager* bm, int32_t num_tokens, int32_t* ok);

/* Prefill of a new sequence: builds its block table from the prompt
 * token_ids[0 .. num_tokens-1] (num_tokens >= 1); *num_cached_tokens receives the
 * prompt tokens whose K/V are already in shared blocks (a multiple of block_size,
 * at most num_tokens - 1).  seq_id must not be live. */
nv_status nv_bm_allocate(nv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                         int32_t num_tokens, int32_t* num_cached_tokens);

/* *ok = 1 if one more token can be appended to seq_id now. */
nv_status nv_bm_can_append(const nv_block_manager* bm, int64_t seq_id, int32_t* ok);

/* Decode: seq_id grows by token_id (may_append: a new block when the token starts
 * one, the last block's hash sealed when the token fills it). */
nv_status nv_bm_append_token(nv_block_manager* bm, int64_t seq_id, int32_t token_id);

/* Ends seq_id and releases its blocks. */
nv_status nv_bm_deallocate(nv_block_manager* bm, int64_t seq_id);

/* Inspection.  nv_bm_get_sequence: *num_tokens, *num_cached_tokens and, if table is
 * not NULL, the block table (capacity entries at most; *num_blocks receives its
 * length).  nv_bm_get_block: the block's reference count, whether it holds a hash
 * and the hash.  nv_bm_get_free_blocks: the free pool front to back. */
nv_status nv_bm_get_sequence(const nv_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                             int32_t* num_cached_tokens, int32_t* table, int32_t capacity,
                             int32_t* num_blocks);
nv_status nv_bm_get_block(const nv_block_manager* bm, int32_t block_id, int32_t* ref_count,
                          int32_t* has_hash, uint64_t* hash);
nv_status nv_bm_get_free_blocks(const nv_block_manager* bm, int32_t* ids, int32_t capacity,
                                int32_t* count);

/* One decode step of `batch` distinct live sequences: appends new_tokens[b] to
 * seq_ids[b], then writes the kernels' metadata for decoding those tokens:
 * block_tables [batch, table_width] (entries past a sequence's blocks = -1),
 * context_lens [batch] (the lengths after the append, the decoded token included)
 * and slot_mapping [batch] (the slot of that token; section 八's block * size +
 * offset).  Capacity and widths are checked before anything changes. */
nv_status nv_bm_decode_step(nv_block_manager* bm, const int64_t* seq_ids,
                            const int32_t* new_tokens, int32_t batch, int32_t* block_tables,
                            int32_t table_width, int32_t* context_lens,
                            int32_t* slot_mapping);

/* One prefill step of num_seqs new sequences: sequence s has the prompt
 * token_ids[cu_tokens[s] .. cu_tokens[s+1]-1] (at least one token).  Allocates them
 * in order and writes block_tables [num_seqs, table_width] (-1 padded) and
 * num_cached [num_seqs]; nv_prepare_prefill then builds cu_seqlens and the slots
 * of the uncached tokens from these.  Capacity (as can_allocate, summed) and
 * widths are checked before anything changes. */
nv_status nv_bm_prefill_step(nv_block_manager* bm, const int64_t* seq_ids,
                             const int32_t* cu_tokens, const int32_t* token_ids,
                             int32_t num_seqs, int32_t* block_tables, int32_t table_width,
                             int32_t* num_cached);

/* XXH64 (seed) of n bytes, the hash the manager uses; exported so that callers and
 * tests can check it against other implementations of the published algorithm. */
uint64_t nv_bm_xxh64(const void* data, int64_t n, uint64_t seed);

#ifdef __cplusplus
}
#endif

#endif /* NVPAGED_BLOCKS_H */
