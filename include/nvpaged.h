/*
 * nvpaged — paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the hot path of a nano-vLLM style engine: the store of new K/V rows
 * into a block-paged cache, paged GQA decode attention and packed varlen causal
 * prefill attention that reads cached prefix blocks, the temperature + Gumbel-max
 * token sampler, plus the host-side metadata builders that produce slot_mapping
 * and cu_seqlens.
 *
 * Sources for the operations (web pages on nano-vLLM):
 *   [walkthrough]  the xingyun3d.csdn.net article on nano-vllm, sections
 *                  五 "KV Block 管理", 六 "模型执行", 七 "后端执行（cuda 算子）",
 *                  八 "序列与上下文";
 *   [paging]       the gsyq.cn article "项目概述：为什么我们需要关注 LLM 推理引擎？",
 *                  sections 4.1 and 5.3;
 *   [deep dive]    "万字深度解析 Nano-vLLM" (chenxutan.com), sections 1.2 and 3.2.1;
 *   [summary]      the gitcode.csdn.net nano-vLLM article, section 三.4.
 *
 * Common conventions
 *   - Cache layout: k_cache and v_cache are each one contiguous device array
 *     [num_blocks, block_size, num_kv_heads, head_dim] in the element dtype.
 *     A slot is the row index into that array viewed as
 *     [num_blocks * block_size, num_kv_heads, head_dim], i.e.
 *     slot = physical_block * block_size + offset ([paging] 4.1, [walkthrough] 八).
 *   - block_tables: int32 [num_seqs, max_blocks_per_seq], row-major; entry i of
 *     row s is the physical block holding tokens i*block_size .. of sequence s.
 *     Entries past a sequence's last used block are never read.
 *   - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads)
 *     ([deep dive] 3.2.1).
 *   - Supported: dtype NV_F32 or NV_BF16 (all tensors of a call share it),
 *     head_dim 64 or 128, block_size a positive multiple of 16,
 *     num_q_heads a multiple of num_kv_heads with at most 8 query heads per KV head.
 *   - Every pointer is caller-owned.  Device pointers must be device memory (for
 *     example from a PyTorch tensor); host pointers are ordinary host memory.
 *     The GPU entry points of this header allocate no memory (the host builders
 *     use temporary host memory) and, with check mode off, keep no state between
 *     calls.  (Check mode keeps a process-wide
 *     switch, a per-thread message and device flags, described with
 *     nv_set_check_mode below.  The host-side block manager of nvpaged_blocks.h
 *     keeps its state in host memory behind a handle the caller creates and
 *     destroys.)
 *   - GPU entry points enqueue work on `stream` (a hipStream_t; NULL = the null
 *     stream) and return without synchronising.  Host-checkable argument errors
 *     are reported before anything is enqueued; a failed launch returns
 *     NV_ERR_HIP.  Values inside device arrays (slots, block ids, lengths) are
 *     preconditions and are not checked: out-of-range values are undefined
 *     behaviour, unless check mode is on (nv_set_check_mode below).
 */
#ifndef NVPAGED_H
#define NVPAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nv_status {
  NV_OK = 0,
  NV_ERR_INVALID_ARG = -1,          /* null pointer, negative size, inconsistent sizes */
  NV_ERR_UNSUPPORTED = -2,          /* head_dim / block_size / dtype / group size not built */
  NV_ERR_WORKSPACE_TOO_SMALL = -3,  /* decode workspace smaller than the size query */
  NV_ERR_HIP = -4,                  /* a HIP launch or runtime call failed */
  NV_ERR_OUT_OF_BLOCKS = -5         /* block manager: too few free blocks (nvpaged_blocks.h) */
} nv_status;

typedef enum nv_dtype {
  NV_F32 = 0,
  NV_BF16 = 1
} nv_dtype;

/* Static, NUL-terminated description of a status code. */
const char* nv_status_string(nv_status status);

/* ------------------------------------------------------------------------- *
 * store_kvcache  ([walkthrough] 七; [summary] 三.4)
 *
 * Before attention, the step's new K/V rows are copied into the pre-allocated
 * cache at the slots given by slot_mapping.  Row i of k (and of v) holds
 * num_kv_heads * head_dim contiguous elements starting at k + i * k_row_stride
 * elements; the stride lets k and v be views into a fused qkv projection.
 * slot_mapping[i] == -1 skips row i (padding) and leaves the cache untouched.
 * The copy is bit-exact.  Non-negative slots must be unique and lie in
 * [0, num_blocks * block_size).  num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------- */
nv_status nv_store_kvcache(const void* k, const void* v,
                           int64_t k_row_stride, int64_t v_row_stride,
                           void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t num_blocks, int32_t block_size,
                           int32_t dtype, void* stream);

/* ------------------------------------------------------------------------- *
 * paged decode  ([walkthrough] 七: decode attends cache_seqlens = context_lens
 * keys through the block table; [deep dive] 1.2: softmax(Q K^T / sqrt(d)) V)
 *
 * out[b, h, :] = softmax(softmax_scale * q[b, h, :] . K_b[t, h/g, :]) V_b[t, h/g, :]
 * over t = 0 .. context_lens[b] - 1, where K_b / V_b are sequence b's rows
 * gathered through block_tables[b].  context_lens[b] counts the token being
 * decoded, whose row must already be stored.
 *   q, out: [batch, num_q_heads, head_dim] contiguous, dtype elements.
 *   context_lens: int32 [batch], each in [1, max_blocks_per_seq * block_size]
 *     and <= max_context_len (a host-side bound used to size the split work).
 *   schedule: optional int32 [batch] device permutation of 0..batch-1 giving
 *     the order in which sequences are started (nv_prepare_decode writes the
 *     length-descending order); NULL = 0..batch-1.  It changes only the order
 *     of work, never the result.
 *   Accumulation is fp32; the output is rounded to the dtype (nearest-even).
 *   workspace: device scratch of at least nv_paged_decode_workspace_size(...)
 *     bytes (may be NULL when that size is 0) for the fp32 partial results of
 *     sequences split into several work items (done when batch * num_kv_heads
 *     is too small to fill the GPU), merged by a second kernel on the same
 *     stream.  No initial contents are required.
 *     Calls that share one workspace must be ordered on one stream.
 *   out must not alias q, the caches or the workspace.  batch == 0 is a no-op.
 * ------------------------------------------------------------------------- */
size_t nv_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len);

nv_status nv_paged_decode(void* out, const void* q,
                          const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, const int32_t* schedule,
                          int32_t max_context_len,
                          int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t num_blocks, int32_t block_size,
                          float softmax_scale, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * fused store + decode: the same result as nv_store_kvcache(k_new, v_new,
 * k_row_stride, v_row_stride, k_cache, v_cache, slot_mapping, batch, ...)
 * followed by nv_paged_decode(...) on the same stream, in one launch (plus the
 * merge launch when sequences are split).  Row b of k_new / v_new is the K/V of
 * sequence b's decoded token; slot_mapping[b] must be the slot of its position
 * context_lens[b] - 1 (as nv_prepare_decode writes it) or -1 to skip the store,
 * in which case that row is read from the cache.  k_new / v_new rows and their
 * strides must be 16-byte aligned (NV_ERR_UNSUPPORTED otherwise).  Each
 * workgroup writes the new row of its own KV head and takes that token's K/V
 * from k_new / v_new, so no read of the written row races the write.
 * ------------------------------------------------------------------------- */
nv_status nv_paged_decode_store(void* out, const void* q,
                                const void* k_new, const void* v_new,
                                int64_t k_row_stride, int64_t v_row_stride,
                                const int32_t* slot_mapping,
                                void* k_cache, void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* schedule,
                                int32_t max_context_len, int32_t batch,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t num_blocks, int32_t block_size,
                                float softmax_scale, int32_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * fused store + decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and launches as
 * nv_paged_decode_store minus the workspace: the fp32 partials of split
 * sequences go to a device array inside the library instead, one copy per GPU
 * of NV_DECODE_STATIC_SCRATCH_BYTES bytes, set up on the first call on that GPU
 * (with that GPU current: the stream must belong to the current device) and
 * held until the process ends.  The call allocates nothing.  It returns
 * NV_ERR_WORKSPACE_TOO_SMALL, before touching the GPU, when the partials would
 * exceed that size (nv_paged_decode_workspace_size(...) > the limit); no plan
 * the kernels support reaches it (head_dim <= 128: the largest split plan's
 * partials take 12.2 MiB, batch 1535 x 8 query heads over one KV head).  The
 * array keeps whatever the last call left; nothing in it needs initial
 * contents.  All calls on one GPU share the array: calls that may overlap (on
 * different streams, or from different host threads without ordering) race
 * and give undefined results; order them on one stream.
 * ------------------------------------------------------------------------- */
#define NV_DECODE_STATIC_SCRATCH_BYTES (16u << 20)

nv_status nv_paged_decode_store_noalloc(void* out, const void* q,
                                        const void* k_new, const void* v_new,
                                        int64_t k_row_stride, int64_t v_row_stride,
                                        const int32_t* slot_mapping,
                                        void* k_cache, void* v_cache,
                                        const int32_t* block_tables,
                                        int32_t max_blocks_per_seq,
                                        const int32_t* context_lens,
                                        const int32_t* schedule,
                                        int32_t max_context_len, int32_t batch,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t num_blocks,
                                        int32_t block_size, float softmax_scale,
                                        int32_t dtype, void* stream);

/* ------------------------------------------------------------------------- *
 * paged varlen prefill  ([walkthrough] 七: the prefill call takes q, the cache,
 * cu_seqlens_q/k, max_seqlen_q/k, causal=True and the block table; 八: only the
 * uncached part of each sequence is computed)
 *
 * Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 (n_s rows)
 * and keys 0 .. k_s-1 with k_s = cu_seqlens_k[s+1] - cu_seqlens_k[s] >= n_s, all
 * read from the cache through block_tables[s] (the new rows must already be
 * stored).  Query row i is the token at position k_s - n_s + i; with causal != 0
 * it attends keys 0 .. k_s - n_s + i (bottom-right aligned mask), otherwise all
 * k_s keys.
 *   q, out: [cu_seqlens_q[num_seqs], num_q_heads, head_dim] contiguous.
 *   cu_seqlens_q/k: int32 [num_seqs + 1], non-decreasing, starting at 0.
 *   max_seqlen_q >= every n_s and max_seqlen_k >= every k_s (host-side bounds
 *   used to size the grid).  Rows of sequences with n_s == 0 are absent.
 *   tile_schedule: optional int32 [2 * num_tiles] device array of (sequence,
 *     query tile) pairs, tile = rows [t * R, (t + 1) * R) with R from
 *     nv_paged_prefill_tile_rows, listing every non-empty tile exactly once;
 *     nv_prepare_prefill writes it heaviest first.  NULL = a dense grid over
 *     max_seqlen_q.  It changes only the order of work, never the result.
 *   out must not alias q or the caches.  num_seqs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
nv_status nv_paged_prefill(void* out, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t max_seqlen_q, int32_t max_seqlen_k,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_seqs,
                           const int32_t* tile_schedule, int32_t num_tiles,
                           int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t num_blocks, int32_t block_size,
                           float softmax_scale, int32_t causal, int32_t dtype,
                           void* stream);

/* Query rows per prefill work tile for this head configuration (0 if unsupported).
 * A tile schedule for nv_paged_prefill is built with this many rows per tile. */
int32_t nv_paged_prefill_tile_rows(int32_t num_q_heads, int32_t num_kv_heads);

/* ------------------------------------------------------------------------- *
 * token sampler  ([walkthrough] 六, sampler paragraph: divide the logits by the
 * temperature, add Gumbel noise, take the argmax; [deep dive] 3.3: temperature 0
 * is greedy decoding)
 *
 * tokens[b] = argmax_i logits[b, i]                         if temperatures[b] == 0
 *           = argmax_i (logits[b, i] / temperatures[b] + gumbel[b, i])  otherwise,
 * with the score computed in binary32 (correctly rounded division, then addition)
 * and ties resolved to the lowest index.  A greedy row never reads its noise row.
 *   tokens: int32 [batch] device output.
 *   logits: [batch, vocab] dtype elements (NV_F32 or NV_BF16), row b starting at
 *     logits + b * logits_row_stride elements.
 *   temperatures: float [batch] device array; each 0 or positive and finite.
 *   gumbel: float [batch, vocab] standard Gumbel(0, 1) draws made by the caller,
 *     row b at gumbel + b * gumbel_row_stride.  Must not be NULL.
 *   NaN logits or noise are undefined behaviour (the result may be out of range).
 *   workspace: 4-byte aligned device scratch of at least
 *     nv_sample_workspace_size(batch, vocab) bytes (NULL allowed when that size
 *     is 0) for per-chunk partial results when rows are split over several
 *     workgroups; merged by a second kernel on the same stream.  No initial
 *     contents are required; calls sharing a workspace must be ordered on one
 *     stream.  batch == 0 is a no-op; batch <= 65535.
 * ------------------------------------------------------------------------- */
size_t nv_sample_workspace_size(int32_t batch, int32_t vocab);

nv_status nv_sample(int32_t* tokens, const void* logits, int64_t logits_row_stride,
                    const float* temperatures, const float* gumbel,
                    int64_t gumbel_row_stride, int32_t batch, int32_t vocab,
                    int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * Check mode.  When on, every GPU entry point above first validates the
 * preconditions on its device arrays with validation kernels on its stream,
 * waits for them (a host synchronisation), and returns NV_ERR_INVALID_ARG
 * without launching its own work if one fails: slots in range and unique
 * (-1 allowed), context lengths within [1, max_context_len] and the table
 * width, block ids of used blocks within [0, num_blocks), a decode schedule that
 * is a permutation, fused-store slots equal to the slot of position
 * context_lens[b] - 1 (or -1), cu_seqlens starting at 0 and non-decreasing
 * with at least as many keys as queries per sequence and within max_seqlen_q/k,
 * a tile schedule listing each existing tile once, sampler temperatures finite
 * and >= 0.  (Uniqueness is checked for arrays of up to 65536 entries; whether
 * a slot lands in a block that several sequences share is not checked.)  Check
 * mode is for debugging: it costs a synchronisation per call and must not be
 * used under stream capture.  It starts on when the environment variable
 * NV_CHECK is set to anything but "0" at the first call, off otherwise.
 * State: the validation kernels report into device-global flags shared by the
 * whole process (one copy per GPU); a process-wide mutex serialises checked
 * calls from the moment the flags are reset until they are read back, so checked
 * calls from several host threads or streams run one after another.  The
 * message is kept per host thread.
 * ------------------------------------------------------------------------- */

/* Turns check mode on (non-zero) or off; returns the previous setting (0 / 1). */
int32_t nv_set_check_mode(int32_t enabled);

/* Description of a violation found by the calling thread's latest check (the
 * lowest-numbered kind found, at its lowest element index; "no violation" if
 * it passed).  Static storage, valid until the
 * thread's next checked call. */
const char* nv_check_message(void);

/* ------------------------------------------------------------------------- *
 * Host-side metadata builders ([walkthrough] 七: prepare_decode /
 * prepare_prefill).  All pointers are HOST memory; nothing touches the GPU.
 * Every block-table entry they read is validated against num_blocks.
 * ------------------------------------------------------------------------- */

/* Decode: slot_mapping[b] = slot of position context_lens[b] - 1 (the token
 * decoded this step); *max_context_len = max_b context_lens[b] (0 if batch == 0).
 * If schedule is not NULL it receives 0..batch-1 in the order nv_paged_decode
 * should start the sequences: first those whose leading block-table entries
 * (within their length) equal another sequence's at the same positions (a shared
 * prefix), more such entries first, then by context length, longest first; ties
 * in index order.  Uses temporary host memory. */
nv_status nv_prepare_decode(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch,
                            int32_t block_size, int32_t num_blocks,
                            int32_t* slot_mapping, int32_t* schedule,
                            int32_t* max_context_len);

/* Prefill: sequence s has num_cached[s] tokens already in the cache and
 * num_new[s] new tokens at positions num_cached[s] .. num_cached[s]+num_new[s]-1.
 * Writes cu_seqlens_q/k ([num_seqs + 1]), the maxima, and the slots of the new
 * tokens in packed order followed by -1 up to the next multiple of pad_to
 * (pad_to >= 1).  slot_capacity is the length of slot_mapping; *num_slots
 * receives the padded count.  If tile_schedule is not NULL it receives the
 * (sequence, tile) pairs of every tile of tile_rows query rows, ordered by
 * causal key count (num_cached + tile end), largest first, ties in order;
 * tile_capacity counts pairs and *num_tiles receives their number.  Returns
 * NV_ERR_INVALID_ARG if something does not fit. */
nv_status nv_prepare_prefill(const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* num_cached, const int32_t* num_new,
                             int32_t num_seqs, int32_t block_size, int32_t num_blocks,
                             int32_t pad_to,
                             int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                             int32_t* max_seqlen_q, int32_t* max_seqlen_k,
                             int32_t* slot_mapping, int32_t slot_capacity,
                             int32_t* num_slots, int32_t tile_rows,
                             int32_t* tile_schedule, int32_t tile_capacity,
                             int32_t* num_tiles);

#ifdef __cplusplus
}
#endif

#endif /* NVPAGED_H */
