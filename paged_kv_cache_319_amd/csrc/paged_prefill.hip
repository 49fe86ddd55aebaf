// Placeholder until the MFMA prefill kernel lands.
#include "common.h"

extern "C" nv_status nv_paged_prefill(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                      int32_t max_seqlen_k, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t num_blocks, int32_t block_size, float softmax_scale,
                                      int32_t causal, int32_t dtype, void* stream) {
  return NV_ERR_UNSUPPORTED;
}
