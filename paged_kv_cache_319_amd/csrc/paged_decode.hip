// Paged GQA decode attention with split-K over fixed token chunks.
//
// Operation (walkthrough, xingyun3d.csdn.net nano-vllm article, section 七;
// softmax(Q K^T / sqrt(d)) V from "万字深度解析 Nano-vLLM", section 1.2): each
// sequence's single query token attends all context_lens[b] keys of its
// sequence, fetched through its block table (paging article on gsyq.cn,
// section 4.1: token t lives in logical block t / B at offset t % B).  Query
// head h reads KV head h / g ("万字深度解析 Nano-vLLM", section 3.2.1).
//
// Work decomposition.  One workgroup (NW waves) handles one (KV head j,
// sequence b, chunk c) triple: tokens [c*CHUNK, (c+1)*CHUNK) of sequence b,
// CHUNK = 64 * NW.  All g query heads of the group are evaluated against every
// K/V row the workgroup loads, so each cached byte is read from HBM once.
// Within a wave a token row of head j (head_dim elements) is spread over LPT
// lanes holding 16 bytes each, so one wave-wide load instruction fetches TPL
// whole rows; every lane issues all of its K and V loads up front (64 tokens
// per wave) to keep many bytes in flight.
//
// Softmax.  Phase 1 forms the scores (v_dot2 for bf16, reductions within the
// LPT-lane groups by DPP), keeps each token's score in exactly one lane, and
// takes the chunk maximum across the waves.  Phase 2 exponentiates once per
// (token, head), publishes the weights through LDS and accumulates P V in fp32.
// Scores carry a log2(e) factor so the exponentials are exp2.
//
// Split merge.  A chunk that covers a whole sequence writes the normalised
// output directly.  Otherwise every chunk writes (m, l, o) partials to the
// workspace and a second, small kernel merges them with log-sum-exp
// rescaling.  (Merging inside the first kernel would need device-scope release
// and acquire fences per workgroup; on this chip those write back and
// invalidate a whole L2 and cost far more than the second launch.)
#include "common.h"

namespace {

using namespace nvp;

constexpr int kDecodeWaves = 4;
constexpr int kDecodeChunk = 64 * kDecodeWaves;  // tokens per workgroup

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;
  float* ws_ml;
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t max_chunks;
  int32_t bs_shift;  // log2(block_size) when it is a power of two, else -1
  float scale_log2;
};

// Logical block of token t (the paging article's t / B).
__device__ __forceinline__ int block_of(int t, const DecodeArgs& a) {
  return a.bs_shift >= 0 ? (t >> a.bs_shift) : (t / a.block_size);
}

template <typename DT, int D, int G, int NW>
__global__ __launch_bounds__(64 * NW) void paged_decode_kernel(DecodeArgs a) {
  using T = typename DT::T;
  constexpr int EPL = DT::kPerLoad;  // elements per 16-byte lane load
  constexpr int LPT = D / EPL;       // lanes per token row
  constexpr int TPL = kWave / LPT;   // token rows per wave load
  constexpr int ITERS = LPT;         // loads per lane: 64 tokens per wave
  constexpr int CHUNK = 64 * NW;
  static_assert(ITERS % 4 == 0, "weights are read four at a time");

  __shared__ float sm_max[NW][G];
  __shared__ float sm_sum[NW][G];
  __shared__ __attribute__((aligned(16))) float sm_p[NW][G][kWave];
  __shared__ float sm_o[NW][G][D];

  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_id();
  const int row = lane / LPT;
  const int col = lane % LPT;
  const int chunk_start = c * CHUNK;
  const int t0 = chunk_start + wave * kWave;

  const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const int32_t* __restrict__ bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const int64_t slot_stride = static_cast<int64_t>(a.num_kv_heads) * D;
  const int64_t head_off = static_cast<int64_t>(j) * D + col * EPL;
  const int qhead0 = j * G;
  const int last_entry = a.max_blocks - 1;

  // The length, this wave's block-table entry and q are independent loads: issue
  // them together.  Table indices are clamped into the row; an entry read for a
  // token at or past the length is never used.
  const int L = a.context_lens[b];
  const bool one_block = a.block_size % kWave == 0;  // the wave's 64 tokens share a block
  const int blk_wave = bt[min(block_of(t0, a), last_entry)];
  u32x4 qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h] = load16(qp + (static_cast<int64_t>(b) * a.num_q_heads + qhead0 + h) * D + col * EPL);
  if (chunk_start >= L) return;  // uniform over the workgroup
  // A length above the host bound max_context_len breaks the contract; clamping keeps
  // every workspace access inside the chunks that were launched.
  const int nchunks = min((L + CHUNK - 1) / CHUNK, a.max_chunks);

  // Issue every K and V load of this lane before any arithmetic.
  u32x4 kr[ITERS], vr[ITERS];
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int tf = t0 + i * TPL;  // first token of this wave load (wave-uniform)
    const int lb = block_of(tf, a);
    const int blk = one_block ? blk_wave : bt[min(lb, last_entry)];
    kr[i] = u32x4{0, 0, 0, 0};
    vr[i] = u32x4{0, 0, 0, 0};
    if (tf + row < L) {
      const int64_t slot = static_cast<int64_t>(blk) * a.block_size + (tf - lb * a.block_size) + row;
      const int64_t e = slot * slot_stride + head_off;
      kr[i] = load16_stream(kc + e);
      vr[i] = load16_stream(vc + e);
    }
  }

  // Phase 1: scores.  After the group reduction all LPT lanes of a row hold the
  // dot product; lane (row, col == i) keeps iteration i's score.
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float part = group_sum<LPT>(dot16<DT>(kr[i], qr[h], 0.f));
      s[h] = (col == i) ? part : s[h];
    }
  }
  const bool valid = (t0 + col * TPL + row) < L;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s[h] = valid ? s[h] * a.scale_log2 : -INFINITY;
    const float wm = group_max<kWave>(s[h]);
    if (lane == 0) sm_max[wave][h] = wm;
  }
  __syncthreads();
  float m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = sm_max[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) x = fmaxf(x, sm_max[w][h]);
    m[h] = x;
  }

  // Phase 2: weights through LDS, then P V.
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float p = valid ? __builtin_amdgcn_exp2f(s[h] - m[h]) : 0.f;
    sm_p[wave][h][lane] = p;
    lsum[h] = group_sum<kWave>(p);
  }
  __builtin_amdgcn_wave_barrier();

  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

#pragma unroll
  for (int i = 0; i < ITERS; i += 4) {
    f32x4 pw[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
      pw[h] = *reinterpret_cast<const f32x4*>(&sm_p[wave][h][row * LPT + i]);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float vv[EPL];
      widen<DT>(vr[i + ii], vv);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw[h][ii], vv[e], acc[h][e]);
    }
  }

  // Fold the TPL rows of the wave, then the waves through LDS.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e]);
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][h][col * EPL + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) sm_sum[wave][h] = lsum[h];
  }
  __syncthreads();

  T* __restrict__ outp = static_cast<T*>(a.out);
  const int64_t qrow0 = static_cast<int64_t>(b) * a.num_q_heads + qhead0;

  if (nchunks == 1) {
    for (int idx = tid; idx < G * D; idx += 64 * NW) {
      const int h = idx / D, d = idx % D;
      float o = 0.f, l = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        o += sm_o[w][h][d];
        l += sm_sum[w][h];
      }
      store_out<DT>(outp + (qrow0 + h) * D + d, o / l);
    }
    return;
  }

  // Partials of this chunk; the merge kernel combines them.
  for (int idx = tid; idx < G * D; idx += 64 * NW) {
    const int h = idx / D, d = idx % D;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      o += sm_o[w][h][d];
      l += sm_sum[w][h];
    }
    const int64_t pidx = (qrow0 + h) * a.max_chunks + c;
    a.ws_o[pidx * D + d] = o;
    if (d == 0) {
      a.ws_ml[pidx * 2] = m[h];
      a.ws_ml[pidx * 2 + 1] = l;
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, query head):
//   M = max_c m_c,  out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c.
// Sequences that fit in one chunk were finished by the attention kernel.
template <typename DT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  using T = typename DT::T;
  constexpr int CHUNK = kDecodeChunk;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int L = a.context_lens[b];
  const int nchunks = min((L + CHUNK - 1) / CHUNK, a.max_chunks);
  if (nchunks <= 1) return;
  const int d = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * a.num_q_heads + h) * a.max_chunks;
  float M = -INFINITY;
  for (int cc = 0; cc < nchunks; ++cc) M = fmaxf(M, a.ws_ml[(base + cc) * 2]);
  float S = 0.f, O = 0.f;
  for (int cc = 0; cc < nchunks; ++cc) {
    const float w = __builtin_amdgcn_exp2f(a.ws_ml[(base + cc) * 2] - M);
    S = fmaf(w, a.ws_ml[(base + cc) * 2 + 1], S);
    O = fmaf(w, a.ws_o[(base + cc) * D + d], O);
  }
  store_out<DT>(static_cast<T*>(a.out) + (static_cast<int64_t>(b) * a.num_q_heads + h) * D + d,
                O / S);
}

struct WsLayout {
  size_t ml_off, o_off, total;
  int max_chunks;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

WsLayout ws_layout(int batch, int hq, int hkv, int d, int max_context_len) {
  WsLayout w{};
  w.max_chunks = max_context_len <= 0 ? 1 : (max_context_len + kDecodeChunk - 1) / kDecodeChunk;
  if (w.max_chunks <= 1) {
    w.total = 0;
    return w;
  }
  w.ml_off = 0;
  w.o_off = w.ml_off + round_up(static_cast<size_t>(batch) * hq * w.max_chunks * 2 * sizeof(float), 256);
  w.total = w.o_off + static_cast<size_t>(batch) * hq * w.max_chunks * d * sizeof(float);
  return w;
}

template <typename DT, int D, int G>
nv_status launch_decode(const DecodeArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.num_kv_heads, batch, a.max_chunks);
  paged_decode_kernel<DT, D, G, kDecodeWaves><<<grid, dim3(64 * kDecodeWaves), 0, s>>>(a);
  if (a.max_chunks > 1)
    decode_merge_kernel<DT, D><<<dim3(a.num_q_heads, batch), dim3(D), 0, s>>>(a);
  return nvp_host::launch_status();
}

template <typename DT, int D>
nv_status dispatch_group(const DecodeArgs& a, int g, int batch, hipStream_t s) {
  switch (g) {
    case 1: return launch_decode<DT, D, 1>(a, batch, s);
    case 2: return launch_decode<DT, D, 2>(a, batch, s);
    case 4: return launch_decode<DT, D, 4>(a, batch, s);
    case 8: return launch_decode<DT, D, 8>(a, batch, s);
    default: return NV_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" size_t nv_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim,
                                                 int32_t max_context_len, int32_t block_size,
                                                 int32_t dtype) {
  (void)block_size;
  (void)dtype;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return ws_layout(batch, num_q_heads, num_kv_heads, head_dim, max_context_len).total;
}

extern "C" nv_status nv_paged_decode(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     int32_t max_context_len, int32_t batch, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                     int32_t block_size, float softmax_scale, int32_t dtype,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return NV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return NV_ERR_INVALID_ARG;
  if (dtype != NV_F32 && dtype != NV_BF16) return NV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return NV_ERR_UNSUPPORTED;
  if (block_size % 16 != 0) return NV_ERR_UNSUPPORTED;
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return NV_ERR_UNSUPPORTED;
  if (batch == 0) return NV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return NV_ERR_INVALID_ARG;
  if (max_context_len < 1 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return NV_ERR_INVALID_ARG;
  if (batch > 65535) return NV_ERR_UNSUPPORTED;
  const WsLayout w = ws_layout(batch, num_q_heads, num_kv_heads, head_dim, max_context_len);
  if (w.max_chunks > 65535) return NV_ERR_UNSUPPORTED;
  if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return NV_ERR_WORKSPACE_TOO_SMALL;

  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  a.ws_ml = w.total ? reinterpret_cast<float*>(ws + w.ml_off) : nullptr;
  a.ws_o = w.total ? reinterpret_cast<float*>(ws + w.o_off) : nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.max_chunks = w.max_chunks;
  a.bs_shift = nvp_host::is_pow2(block_size) ? __builtin_ctz(static_cast<unsigned>(block_size)) : -1;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == NV_BF16) {
    return head_dim == 128 ? dispatch_group<BF16, 128>(a, g, batch, s)
                           : dispatch_group<BF16, 64>(a, g, batch, s);
  }
  return head_dim == 128 ? dispatch_group<F32, 128>(a, g, batch, s)
                         : dispatch_group<F32, 64>(a, g, batch, s);
}
