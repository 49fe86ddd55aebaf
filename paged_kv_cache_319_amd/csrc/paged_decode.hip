// Paged GQA decode attention: length-scheduled work items, wave-local online softmax,
// split-K with a log-sum-exp merge for long contexts.
//
// Operation (walkthrough, xingyun3d.csdn.net nano-vllm article, section 七;
// softmax(Q K^T / sqrt(d)) V from "万字深度解析 Nano-vLLM", section 1.2): each
// sequence's single query token attends all context_lens[b] keys of its
// sequence, fetched through its block table (gsyq.cn paging article, section
// 4.1: token t lives in logical block t / B at offset t % B).  Query head h
// reads KV head h / g ("万字深度解析 Nano-vLLM", section 3.2.1).
//
// Work decomposition.  A work item is (KV head j, sequence b, chunk c): tokens
// [c*chunk, (c+1)*chunk) of sequence b.  The host picks the chunk: whole
// sequences when batch * kv_heads alone fills the chip, otherwise a length
// that yields roughly 2048 items when the longest context is at most 8 K tokens and
// 512 above (at least two chunks per sequence).
// Sequences are visited in the order of an optional schedule (the host's
// length-descending order from nv_prepare_decode), so the longest items start
// first and the short ones fill the tail.  The NW waves of a KV head walk its
// item in passes of TPW*NW tokens; every lane issues all of its K and V loads of
// a pass (4 + 4 non-temporal 16-byte loads for bf16, head_dim 128: 16 tokens per
// wave) before any arithmetic.  Short passes keep the kernel small (~80-100
// VGPRs): while one wave computes, the others on the CU still have loads in
// flight (batch-256 step: 64-token passes 92 us, 32-token 89.6 us, 16-token
// 87.7 us, event-timed).  A workgroup holds one or two KV heads and 16 waves
// share a CU; the shapes per plan are chosen in launch_decode.
//
// Lanes.  A token row of head j (head_dim elements) is spread over LPT lanes of
// 16 bytes, so one wave-wide load fetches TPL whole rows.  The g query heads of
// the group are evaluated against every loaded row: each cached byte is read
// from HBM once per step.
//
// Softmax.  Per pass: scores (v_dot2 for bf16, DPP reductions within LPT-lane
// groups), each token's score kept in exactly one lane, the wave's pass maximum,
// then an online update of the wave's own state (running max m, sum l and P V
// accumulator rescaled by 2^(m_old - m_new)).  The waves never wait for each other
// inside the pass loop; their states are merged once at the end, each weighted by
// 2^(m_wave - M).  Weights reach the P V loop through LDS.  Scores carry a log2(e)
// factor so the exponentials are exp2.
//
// Split merge.  A chunk that covers a whole sequence writes the normalised
// output.  Otherwise each chunk writes (m, l, o) partials to the workspace and
// a second, small kernel merges them.  (Merging inside the first kernel needs
// device-scope release/acquire fences per workgroup; on this chip each writes
// back and invalidates a whole L2 and costs far more than the second launch.)
#include <algorithm>
#include <mutex>

#include "common.h"

namespace {

using namespace nvp;

constexpr int kDecodeWaves = 4;
constexpr int kPass = 256;                // chunk granularity (a multiple of every pass)
constexpr int kSplitBelowItems = 1536;    // split sequences when fewer (head, sequence) items
// Work items aimed at when splitting (>= 2 chunks per sequence): more, shorter chunks
// balance ragged contexts up to 8 K tokens (batch 64 x U[128, 4096]: 1.5 % faster with
// 2048 than with 512); at 32 K tokens the extra chunks cost more in merging (-5.8 %).
constexpr int kTargetSplitItemsShort = 2048;
constexpr int kTargetSplitItemsLong = 512;
constexpr int kShortContext = 8192;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* schedule;  // sequence visiting order, or null for 0..batch-1
  // Fused store (nv_paged_decode_store): this step's K/V rows and their slots.
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
  int64_t k_new_stride;     // elements between rows of k_new / v_new
  int64_t v_new_stride;
  float* ws_o;
  float* ws_ml;
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t chunk;            // tokens per work item, a multiple of kPass
  int32_t max_chunks;
  int32_t bs_shift;         // log2(block_size) when it is a power of two, else -1
  float scale_log2;
};

// Token rows one wave covers per pass: LPT = D / (16 / sizeof(T)) lanes hold one row,
// a wave load covers 64 / LPT rows, and each lane issues max(LPT / 4, 4) loads.
template <typename DT, int D>
constexpr int decode_tokens_per_wave_pass() {
  return (D / DT::kPerLoad >= 16 ? D / DT::kPerLoad / 4 : 4) * (kWave / (D / DT::kPerLoad));
}

// Logical block of token t (the paging article's t / B).  FAST: the block size is a
// power of two no smaller than the tokens of a wave-pass; passes start at multiples of
// that count, so a wave-pass never straddles a block and needs one table entry.
template <bool FAST>
__device__ __forceinline__ int block_of(int t, const DecodeArgs& a) {
  return FAST ? (t >> a.bs_shift) : (t / a.block_size);
}

// Returns x unchanged, held in a vector register: the compiler then treats it as
// varying over the wave, so a load from an address built on it is a vector memory load
// rather than a scalar one.  Used for the per-pass block-table entry, which measured
// faster through the vector path (4 % on the 32 K-context split decode).
__device__ __forceinline__ int in_vgpr(int x) {
  asm("" : "+v"(x));
  return x;
}

// One workgroup = HPW KV heads (blockIdx.x * HPW ..) of one (sequence, chunk) item, NW
// waves per head splitting the item's tokens; the heads' waves share nothing but the
// workgroup, so its rows of consecutive heads are read side by side.
template <typename DT, int D, int G, int NW, bool FAST, bool STORE, int HPW>
__global__ __launch_bounds__(64 * NW * HPW) void paged_decode_kernel(DecodeArgs a) {
  using T = typename DT::T;
  constexpr int EPL = DT::kPerLoad;  // elements per 16-byte lane load
  constexpr int LPT = D / EPL;       // lanes per token row
  constexpr int TPL = kWave / LPT;   // token rows per wave load
  constexpr int ITERS = LPT >= 16 ? LPT / 4 : 4;  // loads per lane per pass (K and V each)
  constexpr int TPW = ITERS * TPL;   // tokens per wave per pass: 16 or 32
  static_assert(TPW == decode_tokens_per_wave_pass<DT, D>(), "pass geometry");
  constexpr int PASS = TPW * NW;
  static_assert(ITERS % 4 == 0 && kWave % TPW == 0, "weights are read four at a time");

  __shared__ float sm_m[NW * HPW][G];
  __shared__ float sm_sum[NW * HPW][G];
  __shared__ __attribute__((aligned(16))) float sm_p[NW * HPW][G][kWave];
  __shared__ float sm_o[NW * HPW][G][D];

  const int wave_all = wave_id();              // 0 .. NW * HPW - 1
  const int j = blockIdx.x * HPW + wave_all / NW;  // this wave's KV head
  const int b = a.schedule ? a.schedule[blockIdx.y] : static_cast<int>(blockIdx.y);
  const int c = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_all % NW;              // index among the head's waves
  const int row = lane / LPT;
  const int col = lane % LPT;

  const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const int32_t* __restrict__ bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const int64_t slot_stride = static_cast<int64_t>(a.num_kv_heads) * D;
  const int64_t head_off = static_cast<int64_t>(j) * D + col * EPL;
  const int qhead0 = j * G;
  const int last_entry = a.max_blocks - 1;
  const int cs = c * a.chunk;

  // The length, the first block-table entry and q are independent loads: issue
  // them together.  Table indices are clamped into the row; an entry read for a
  // token at or past the length is never used.
  const int L = a.context_lens[b];
  const int slot_new = STORE ? a.new_slots[b] : -1;
  int blk_wave = bt[min(block_of<FAST>(cs + wave * TPW, a), last_entry)];
  u32x4 qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h] = load16(qp + (static_cast<int64_t>(b) * a.num_q_heads + qhead0 + h) * D + col * EPL);
  if (cs >= L) return;  // uniform over the workgroup
  const int ce = min(L, cs + a.chunk);
  // A length above the host bound max_context_len breaks the contract; clamping keeps
  // every workspace access inside the chunks that were launched.
  const int nchunks = min((L + a.chunk - 1) / a.chunk, a.max_chunks);

  // Fused store: the K/V row of the decoded token (position L - 1) comes from this
  // step's input.  In the chunk that holds it, row 0 of wave 0 loads that row of head j
  // here, and after the loop writes it to its cache slot and adds the token to wave 0's
  // softmax state; the loop itself covers the cached tokens [cs, ce_c) only.  No other
  // workgroup reads that row of head j, so the write races no read.
  const int pos_new = (STORE && slot_new >= 0) ? L - 1 : -1;
  const bool new_here = STORE && pos_new >= cs && pos_new < ce;
  const int ce_c = new_here ? pos_new : ce;
  u32x4 kn_r = u32x4{0, 0, 0, 0}, vn_r = u32x4{0, 0, 0, 0};
  if (new_here && wave == 0 && row == 0) {
    kn_r = load16(static_cast<const T*>(a.k_new) + static_cast<int64_t>(b) * a.k_new_stride + head_off);
    vn_r = load16(static_cast<const T*>(a.v_new) + static_cast<int64_t>(b) * a.v_new_stride + head_off);
  }

  float m_run[G], l_run[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  for (int ps = cs; ps < ce_c; ps += PASS) {
    const int t0 = ps + wave * TPW;
    if (t0 >= ce_c) break;  // wave-uniform; the loop has no workgroup barrier
    if (ps != cs) blk_wave = bt[in_vgpr(min(block_of<FAST>(t0, a), last_entry))];

    // Issue every K and V load of this pass before any arithmetic.
    u32x4 kr[ITERS], vr[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int tf = t0 + i * TPL;  // first token of this wave load (wave-uniform)
      int blk, off;
      if constexpr (FAST) {
        blk = blk_wave;
        off = tf & (a.block_size - 1);
      } else {
        const int lb = block_of<FAST>(tf, a);
        blk = bt[min(lb, last_entry)];
        off = tf - lb * a.block_size;
      }
      kr[i] = u32x4{0, 0, 0, 0};
      vr[i] = u32x4{0, 0, 0, 0};
      if (tf + row < ce_c) {
        const int64_t slot = static_cast<int64_t>(blk) * a.block_size + off + row;
        const int64_t e = slot * slot_stride + head_off;
        kr[i] = load16_stream(kc + e);
        vr[i] = load16_stream(vc + e);
      }
    }
    // Scores.  After the group reduction all LPT lanes of a row hold the dot
    // product; lane (row, col == i) keeps iteration i's score (lanes with
    // col >= ITERS keep none).
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
    const bool valid = col < ITERS && (t0 + col * TPL + row) < ce_c;
    // Online softmax per wave: the pass maximum of this wave (finite: its first token
    // is valid).  The running maximum moves only when a pass exceeds it by more than 8
    // (weights stay at most 2^8), so the rescale of the accumulators is rare; the waves'
    // states are combined once, at the end.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] = valid ? s[h] * a.scale_log2 : -INFINITY;
      const float wm = group_max<kWave>(s[h]);
      const float m_use = wm > m_run[h] + 8.f ? wm : m_run[h];
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_use);
      m_run[h] = m_use;
      const float p = valid ? __builtin_amdgcn_exp2f(s[h] - m_use) : 0.f;
      sm_p[wave_all][h][lane] = p;
      l_run[h] = l_run[h] * alpha + p;
      if (alpha != 1.f) {  // wave-uniform
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
      }
    }
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int i = 0; i < ITERS; i += 4) {
      f32x4 pw[G];
#pragma unroll
      for (int h = 0; h < G; ++h)
        pw[h] = *reinterpret_cast<const f32x4*>(&sm_p[wave_all][h][row * LPT + i]);
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
    __builtin_amdgcn_wave_barrier();  // sm_p is rewritten by the next pass
  }

  if (new_here && wave == 0) {  // wave-uniform: the decoded token
    if (row == 0) {
      const int64_t e = static_cast<int64_t>(slot_new) * slot_stride + head_off;
      *reinterpret_cast<u32x4*>(const_cast<T*>(kc) + e) = kn_r;
      *reinterpret_cast<u32x4*>(const_cast<T*>(vc) + e) = vn_r;
    }
    float vv[EPL];
    widen<DT>(vn_r, vv);  // zero outside row 0
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // Row 0 holds the score after the group reduction; lane 0 broadcasts it.
      const float part = group_sum<LPT>(dot16<DT>(kn_r, qr[h], 0.f)) * a.scale_log2;
      const float sn = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(part)));
      const float m_new = fmaxf(m_run[h], sn);
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);  // 0 if no cached token
      const float p = __builtin_amdgcn_exp2f(sn - m_new);
      m_run[h] = m_new;
      l_run[h] = l_run[h] * alpha + (lane == 0 ? p : 0.f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vv[e], acc[h][e] * alpha);
    }
  }

  // Fold the TPL rows of each wave, then the waves through LDS, each weighted by
  // 2^(m_wave - M) with M the largest wave maximum.  A wave that saw no token holds
  // m = -inf and zero sums (weight 0); wave 0 always holds a token: the chunk's first
  // cached one, or the decoded one when that is the chunk's only token.
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = group_sum<kWave>(l_run[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e]);
  }
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave_all][h][col * EPL + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_sum[wave_all][h] = lsum[h];
      sm_m[wave_all][h] = m_run[h];
    }
  }
  __syncthreads();

  T* __restrict__ outp = static_cast<T*>(a.out);
  for (int idx = tid; idx < HPW * G * D; idx += 64 * NW * HPW) {
    const int hs = idx / (G * D), h = (idx / D) % G, d = idx % D;
    const int64_t qrow0 =
        static_cast<int64_t>(b) * a.num_q_heads + (blockIdx.x * HPW + hs) * G;
    const int w0 = hs * NW;                    // the waves of KV head blockIdx.x*HPW + hs
    float M = sm_m[w0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w0 + w][h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[w0 + w][h] - M);
      o = fmaf(f, sm_o[w0 + w][h][d], o);
      l = fmaf(f, sm_sum[w0 + w][h], l);
    }
    if (nchunks == 1) {
      store_out<DT>(outp + (qrow0 + h) * D + d, o / l);
    } else {
      const int64_t pidx = (qrow0 + h) * a.max_chunks + c;
      a.ws_o[pidx * D + d] = o;
      if (d == 0) {
        a.ws_ml[pidx * 2] = M;
        a.ws_ml[pidx * 2 + 1] = l;
      }
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, query head):
//   M = max_c m_c,  out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c.
// Sequences that fit in one chunk were finished by the attention kernel.
template <typename DT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  using T = typename DT::T;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int L = a.context_lens[b];
  const int nchunks = min((L + a.chunk - 1) / a.chunk, a.max_chunks);
  if (nchunks <= 1) return;
  const int d = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * a.num_q_heads + h) * a.max_chunks;
  // Groups of up to eight chunks: every load of a group is issued before any arithmetic
  // (one memory round trip per group), then the group's maximum, the rescale of the sums
  // so far (by 0 on the first group) and the weighted sums in chunk order.
  constexpr int kGroup = 8;
  float M = -INFINITY, S = 0.f, O = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += kGroup) {
    float m[kGroup], l[kGroup], o[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int cc = min(c0 + j, nchunks - 1);
      const bool live = c0 + j < nchunks;
      const float mv = a.ws_ml[(base + cc) * 2];
      const float lv = a.ws_ml[(base + cc) * 2 + 1];
      const float ov = a.ws_o[(base + cc) * D + d];
      m[j] = live ? mv : -INFINITY;
      l[j] = live ? lv : 0.f;
      o[j] = live ? ov : 0.f;
    }
    float Mg = M;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) Mg = fmaxf(Mg, m[j]);
    const float r = __builtin_amdgcn_exp2f(M - Mg);   // M = -inf on the first group: 0
    S *= r;
    O *= r;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float w = __builtin_amdgcn_exp2f(m[j] - Mg);
      S = fmaf(w, l[j], S);
      O = fmaf(w, o[j], O);
    }
    M = Mg;
  }
  store_out<DT>(static_cast<T*>(a.out) + (static_cast<int64_t>(b) * a.num_q_heads + h) * D + d,
                O / S);
}

// Host-side plan: tokens per work item and the resulting workspace layout.
struct Plan {
  int chunk, max_chunks;
  size_t ml_off, o_off, total;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Plan make_plan(int batch, int hq, int hkv, int d, int max_context_len) {
  Plan p{};
  const int max_len = max_context_len < 1 ? 1 : max_context_len;
  const int64_t items = static_cast<int64_t>(batch) * hkv;
  int64_t per_seq = 1;  // chunks per sequence
  if (items < kSplitBelowItems) {
    const int64_t target = max_len <= kShortContext ? kTargetSplitItemsShort : kTargetSplitItemsLong;
    per_seq = std::max<int64_t>(2, (target + items - 1) / items);
  }
  int64_t chunk = (max_len + per_seq - 1) / per_seq;
  chunk = static_cast<int64_t>(round_up(static_cast<size_t>(chunk), kPass));
  p.chunk = static_cast<int>(chunk);
  p.max_chunks = static_cast<int>((max_len + chunk - 1) / chunk);
  if (p.max_chunks <= 1) {
    p.total = 0;
    return p;
  }
  p.ml_off = 0;
  p.o_off = round_up(static_cast<size_t>(batch) * hq * p.max_chunks * 2 * sizeof(float), 256);
  p.total = p.o_off + static_cast<size_t>(batch) * hq * p.max_chunks * d * sizeof(float);
  return p;
}

// Shared memory of the arrays of one KV head's NW waves in a decode workgroup.
template <int D, int G, int NW>
constexpr size_t decode_static_lds() {
  return sizeof(float) * (2 * NW * G + NW * G * kWave + NW * G * D);
}
// Workgroup shape by plan (measured on the batch-256, batch-64 and 32K-context
// workloads).  Every sequence one work item: two KV heads per workgroup, 4 waves per
// head, 72 KB of LDS reserved (two workgroups, 16 waves per CU; fewer concurrent streams
// read the head-strided rows of whole sequences best, and the two heads' rows sit side
// by side); one head of 4 waves with 36 KB when the KV-head count is odd.  Sequences
// split into chunks: one head of 8 waves per workgroup (each chunk finishes in half the
// time, which evens out the few items per resident workgroup such plans have), 56 KB
// reserved (two per CU, the same 16 waves).
constexpr size_t kDecodeLdsPerWorkgroup = 36 * 1024;
constexpr size_t kDecodeLdsPerWorkgroupPair = 72 * 1024;
constexpr int kDecodeWavesSplit = 8;
constexpr size_t kDecodeLdsPerWorkgroupSplit = 56 * 1024;

template <typename DT, int D, int G, int NW, int HPW, size_t LDS_CAP>
void launch_decode_kernel(const DecodeArgs& a, int batch, hipStream_t s) {
  static_assert(HPW * decode_static_lds<D, G, NW>() <= LDS_CAP, "LDS");
  const dim3 grid(a.num_kv_heads / HPW, batch, a.max_chunks);
  const dim3 block(64 * NW * HPW);
  const size_t pad = LDS_CAP - HPW * decode_static_lds<D, G, NW>();
  const bool fast = a.bs_shift >= 0 && (1 << a.bs_shift) >= decode_tokens_per_wave_pass<DT, D>();
  if (a.new_slots) {
    if (fast) paged_decode_kernel<DT, D, G, NW, true, true, HPW><<<grid, block, pad, s>>>(a);
    else paged_decode_kernel<DT, D, G, NW, false, true, HPW><<<grid, block, pad, s>>>(a);
  } else {
    if (fast) paged_decode_kernel<DT, D, G, NW, true, false, HPW><<<grid, block, pad, s>>>(a);
    else paged_decode_kernel<DT, D, G, NW, false, false, HPW><<<grid, block, pad, s>>>(a);
  }
}

template <typename DT, int D, int G>
nv_status launch_decode(const DecodeArgs& a, int batch, hipStream_t s) {
  if (a.max_chunks > 1) {
    launch_decode_kernel<DT, D, G, kDecodeWavesSplit, 1, kDecodeLdsPerWorkgroupSplit>(a, batch, s);
    decode_merge_kernel<DT, D><<<dim3(a.num_q_heads, batch), dim3(D), 0, s>>>(a);
  } else if (a.num_kv_heads % 2 == 0) {
    launch_decode_kernel<DT, D, G, kDecodeWaves, 2, kDecodeLdsPerWorkgroupPair>(a, batch, s);
  } else {
    launch_decode_kernel<DT, D, G, kDecodeWaves, 1, kDecodeLdsPerWorkgroup>(a, batch, s);
  }
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
                                                 int32_t max_context_len) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return make_plan(batch, num_q_heads, num_kv_heads, head_dim, max_context_len).total;
}

namespace {

nv_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, const int32_t* schedule,
                      int32_t max_context_len, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                      int32_t block_size, float softmax_scale, int32_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream, const void* k_new, const void* v_new,
                      int64_t k_new_stride, int64_t v_new_stride, const int32_t* new_slots) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return NV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return NV_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY ||
      softmax_scale == -INFINITY)
    return NV_ERR_INVALID_ARG;
  if (dtype != NV_F32 && dtype != NV_BF16) return NV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return NV_ERR_UNSUPPORTED;
  if (block_size % 16 != 0) return NV_ERR_UNSUPPORTED;
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return NV_ERR_UNSUPPORTED;
  if (batch == 0) return NV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return NV_ERR_INVALID_ARG;
  if (new_slots) {
    const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
    const int64_t esize = dtype == NV_F32 ? 4 : 2;
    if (!k_new || !v_new || k_new_stride < row || v_new_stride < row) return NV_ERR_INVALID_ARG;
    const uintptr_t align = reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                            static_cast<uintptr_t>(k_new_stride * esize) |
                            static_cast<uintptr_t>(v_new_stride * esize);
    if (align & 15) return NV_ERR_UNSUPPORTED;  // rows are moved as 16-byte pieces
  }
  if (max_context_len < 1 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return NV_ERR_INVALID_ARG;
  if (batch > 65535) return NV_ERR_UNSUPPORTED;
  const Plan p = make_plan(batch, num_q_heads, num_kv_heads, head_dim, max_context_len);
  if (p.max_chunks > 65535) return NV_ERR_UNSUPPORTED;
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return NV_ERR_WORKSPACE_TOO_SMALL;
  if (nvp_check::on()) {
    const nv_status st = nvp_check::decode(block_tables, max_blocks_per_seq, context_lens, schedule,
                                           new_slots, batch, block_size, num_blocks,
                                           max_context_len, stream);
    if (st != NV_OK) return st;
  }

  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.schedule = schedule;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_slots = new_slots;
  a.k_new_stride = k_new_stride;
  a.v_new_stride = v_new_stride;
  char* ws = static_cast<char*>(workspace);
  a.ws_ml = p.total ? reinterpret_cast<float*>(ws + p.ml_off) : nullptr;
  a.ws_o = p.total ? reinterpret_cast<float*>(ws + p.o_off) : nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.chunk = p.chunk;
  a.max_chunks = p.max_chunks;
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

}  // namespace

extern "C" nv_status nv_paged_decode(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     const int32_t* schedule, int32_t max_context_len,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_blocks, int32_t block_size,
                                     float softmax_scale, int32_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     schedule, max_context_len, batch, num_q_heads, num_kv_heads, head_dim,
                     num_blocks, block_size, softmax_scale, dtype, workspace, workspace_bytes,
                     stream, nullptr, nullptr, 0, 0, nullptr);
}

extern "C" nv_status nv_paged_decode_store(void* out, const void* q, const void* k_new,
                                           const void* v_new, int64_t k_row_stride,
                                           int64_t v_row_stride, const int32_t* slot_mapping,
                                           void* k_cache, void* v_cache,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, const int32_t* schedule,
                                           int32_t max_context_len, int32_t batch,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t num_blocks,
                                           int32_t block_size, float softmax_scale, int32_t dtype,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && !slot_mapping) return NV_ERR_INVALID_ARG;
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     schedule, max_context_len, batch, num_q_heads, num_kv_heads, head_dim,
                     num_blocks, block_size, softmax_scale, dtype, workspace, workspace_bytes,
                     stream, k_new, v_new, k_row_stride, v_row_stride,
                     batch > 0 ? slot_mapping : nullptr);
}

// ---------------------------------------------------------------------------
// Allocation-free variant of the fused store + decode.  The split-K partials live
// in `scratch`, a device array of this file (one copy per GPU, held until the
// process ends) instead of a caller workspace.  Host code never passes the array's
// name to a kernel (in host code it is only a stand-in for the symbol): the device
// address is looked up once per GPU, with that GPU current, and kept.
// ---------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[NV_DECODE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current GPU (set up on the first call there).
nv_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return NV_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return NV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return NV_OK;
}

}  // namespace

extern "C" nv_status nv_paged_decode_store_noalloc(
    void* out, const void* q, const void* k_new, const void* v_new, int64_t k_row_stride,
    int64_t v_row_stride, const int32_t* slot_mapping, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* schedule, int32_t max_context_len, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
    float softmax_scale, int32_t dtype, void* stream) {
  if (batch > 0 && !slot_mapping) return NV_ERR_INVALID_ARG;
  // Partials this call needs (0 when no sequence is split); decided before any GPU call.
  const size_t need = nv_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                     max_context_len);
  if (need > NV_DECODE_STATIC_SCRATCH_BYTES) return NV_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    const nv_status st = scratch_for_current_device(&ws);
    if (st != NV_OK) return st;
  }
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     schedule, max_context_len, batch, num_q_heads, num_kv_heads, head_dim,
                     num_blocks, block_size, softmax_scale, dtype, ws,
                     need > 0 ? static_cast<size_t>(NV_DECODE_STATIC_SCRATCH_BYTES) : 0, stream,
                     k_new, v_new, k_row_stride, v_row_stride,
                     batch > 0 ? slot_mapping : nullptr);
}
