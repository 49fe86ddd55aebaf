// Token sampler: temperature scaling + Gumbel-max, one token per row of logits.
//
// Walkthrough (xingyun3d.csdn.net nano-vllm article), section 六, sampler
// paragraph: the logits are divided by the temperature, noise is added and the
// argmax is the sampled token, a sort-free parallel form of drawing from
// softmax(logits / T).  Deep dive ("万字深度解析 Nano-vLLM") section 3.3:
// temperature 0 is greedy decoding.  The Gumbel draws are an input.
//
// The work is one streaming pass over [batch, vocab] logits (and the noise of
// rows with T > 0), so it is bound by HBM bandwidth.  Each row is cut into
// `chunks` contiguous pieces (one piece per row when the batch alone fills the
// chip); workgroup (chunk, row) streams its piece with 16-byte non-temporal loads,
// eight elements per lane and step, keeps the best (score, index) per lane and
// reduces it over the workgroup.  With one chunk per row the workgroup writes the
// token; otherwise it writes a partial pair and a second kernel reduces the chunks
// of each row.
//
// Scores are binary32: s = (z / T) + g, with a correctly rounded division and
// addition, so the argmax is a well-defined function of the inputs.  Ties go to
// the lowest index.  Greedy rows (T == 0) compare the raw logits and never read
// their noise row.
#include <math.h>

#include "common.h"

namespace {

constexpr int kThreads = 256;  // split plans and the merge kernel
constexpr int kUnit = 8;       // elements per lane-step
constexpr int kUnroll = 4;     // split plans: lane-steps whose loads are issued together
// Batches of at least kRowPlanBatch rows: one kRowThreads-thread workgroup per row
// (enough rows to fill the chip), kRowUnroll lane-steps in flight, no merge.
constexpr int kRowPlanBatch = 256;
constexpr int kRowThreads = 1024;
constexpr int kRowUnroll = 2;

struct Best {
  float s;
  int32_t i;
};

// (s, i) beats (t, j): higher score, or the same score at a lower index.  NaN
// scores never win.
__device__ __forceinline__ bool better(float s, int32_t i, float t, int32_t j) {
  return s > t || (s == t && i < j);
}

__device__ __forceinline__ void take(Best& b, float s, int32_t i) {
  if (better(s, i, b.s, b.i)) {
    b.s = s;
    b.i = i;
  }
}

__device__ __forceinline__ Best wave_best(Best b) {
#pragma unroll
  for (int m = 1; m < nvp::kWave; m <<= 1) {
    const float s = __shfl_xor(b.s, m, nvp::kWave);
    const int32_t i = __shfl_xor(b.i, m, nvp::kWave);
    take(b, s, i);
  }
  return b;
}

// Best over the workgroup of NT threads; the result is valid in thread 0.
template <int NT>
__device__ __forceinline__ Best block_best(Best b) {
  __shared__ float ss[NT / nvp::kWave];
  __shared__ int32_t si[NT / nvp::kWave];
  b = wave_best(b);
  const int w = threadIdx.x / nvp::kWave;
  if ((threadIdx.x & (nvp::kWave - 1)) == 0) {
    ss[w] = b.s;
    si[w] = b.i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 1; k < NT / nvp::kWave; ++k) take(b, ss[k], si[k]);
  }
  return b;
}

// Eight logits of one lane-step as floats.
template <typename DT>
struct Logits8;

template <>
struct Logits8<nvp::BF16> {
  nvp::u32x4 r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = nvp::load16_stream(p); }
  __device__ __forceinline__ float at(int e) const {
    const uint32_t w = r[e >> 1];
    return (e & 1) ? nvp::bf16_hi(w) : nvp::bf16_lo(w);
  }
};

template <>
struct Logits8<nvp::F32> {
  nvp::u32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = nvp::load16_stream(p);
    b = nvp::load16_stream(p + 4);
  }
  __device__ __forceinline__ float at(int e) const {
    const uint32_t w = e < 4 ? a[e & 3] : b[e & 3];
    return __uint_as_float(w);
  }
};

struct Noise8 {
  nvp::u32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = nvp::load16_stream(p);
    b = nvp::load16_stream(p + 4);
  }
  __device__ __forceinline__ float at(int e) const {
    const uint32_t w = e < 4 ? a[e & 3] : b[e & 3];
    return __uint_as_float(w);
  }
};

template <bool GREEDY>
__device__ __forceinline__ float score(float z, float t, float g) {
  if constexpr (GREEDY)
    return z;
  else
    return __fdiv_rn(z, t) + g;
}

// Best (score, index) of one lane over elements lo .. hi-1 of a row.  A lane
// visits its elements in increasing index order, so a strict comparison keeps the
// first of equal scores; a lane whose scores are all -inf reports its first index.
// VEC: row bases and strides are 16-byte aligned, so lane-steps of eight elements
// are read with 16-byte loads; otherwise every element is loaded on its own.
template <typename DT, bool VEC, bool GREEDY, int NT, int UNROLL>
__device__ __forceinline__ Best scan(const typename DT::T* __restrict__ zr,
                                     const float* __restrict__ gr, float t, int32_t lo,
                                     int32_t hi) {
  float bs = -INFINITY;
  int32_t bi = INT32_MAX;
  int32_t first = INT32_MAX;
  int32_t tail = lo;  // first element not covered by whole lane-steps
  if constexpr (VEC) {
    const int32_t steps = (hi - lo) / kUnit;
    tail = lo + steps * kUnit;
    int32_t u = threadIdx.x;
    if (u < steps) first = lo + u * kUnit;
    for (; u + (UNROLL - 1) * NT < steps; u += UNROLL * NT) {
      Logits8<DT> z[UNROLL];
      Noise8 g[UNROLL];
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) z[k].load(zr + lo + (u + k * NT) * kUnit);
      if constexpr (!GREEDY) {
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) g[k].load(gr + lo + (u + k * NT) * kUnit);
      }
#pragma unroll
      for (int k = 0; k < UNROLL; ++k) {
        const int32_t base = lo + (u + k * NT) * kUnit;
#pragma unroll
        for (int e = 0; e < kUnit; ++e) {
          const float s = score<GREEDY>(z[k].at(e), t, GREEDY ? 0.0f : g[k].at(e));
          const bool win = s > bs;
          bs = win ? s : bs;
          bi = win ? base + e : bi;
        }
      }
    }
    for (; u < steps; u += NT) {
      Logits8<DT> z;
      Noise8 g;
      z.load(zr + lo + u * kUnit);
      if constexpr (!GREEDY) g.load(gr + lo + u * kUnit);
      const int32_t base = lo + u * kUnit;
#pragma unroll
      for (int e = 0; e < kUnit; ++e) {
        const float s = score<GREEDY>(z.at(e), t, GREEDY ? 0.0f : g.at(e));
        const bool win = s > bs;
        bs = win ? s : bs;
        bi = win ? base + e : bi;
      }
    }
  }
  if (first == INT32_MAX && tail + static_cast<int32_t>(threadIdx.x) < hi)
    first = tail + threadIdx.x;
  for (int32_t i = tail + threadIdx.x; i < hi; i += NT) {
    float z;
    if constexpr (sizeof(typename DT::T) == 2)
      z = nvp::bf16_lo(static_cast<uint32_t>(zr[i]));
    else
      z = zr[i];
    const float s = score<GREEDY>(z, t, GREEDY ? 0.0f : gr[i]);
    const bool win = s > bs;
    bs = win ? s : bs;
    bi = win ? i : bi;
  }
  if (bi == INT32_MAX) bi = first;
  return Best{bs, bi};
}

template <typename DT, bool VEC, int NT, int UNROLL>
__global__ __launch_bounds__(NT) void sample_partial_kernel(
    const typename DT::T* __restrict__ logits, int64_t logits_stride,
    const float* __restrict__ temperatures, const float* __restrict__ gumbel,
    int64_t gumbel_stride, int32_t vocab, int32_t chunk, int32_t chunks,
    float* __restrict__ part_score, int32_t* __restrict__ part_index,
    int32_t* __restrict__ tokens) {
  const int32_t row = blockIdx.y;
  const int32_t c = blockIdx.x;
  const int32_t lo = c * chunk;
  const int32_t hi = static_cast<int32_t>(
      min(static_cast<int64_t>(vocab), static_cast<int64_t>(lo) + chunk));
  const float t = temperatures[row];
  const typename DT::T* zr = logits + static_cast<int64_t>(row) * logits_stride;
  const float* gr = gumbel + static_cast<int64_t>(row) * gumbel_stride;
  Best best = t == 0.0f ? scan<DT, VEC, true, NT, UNROLL>(zr, gr, t, lo, hi)
                        : scan<DT, VEC, false, NT, UNROLL>(zr, gr, t, lo, hi);
  best = block_best<NT>(best);
  if (threadIdx.x == 0) {
    if (chunks == 1) {
      tokens[row] = best.i;
    } else {
      part_score[static_cast<int64_t>(row) * chunks + c] = best.s;
      part_index[static_cast<int64_t>(row) * chunks + c] = best.i;
    }
  }
}

// One wave per row reduces the row's chunk partials.
__global__ __launch_bounds__(kThreads) void sample_merge_kernel(
    const float* __restrict__ part_score, const int32_t* __restrict__ part_index,
    int32_t chunks, int32_t batch, int32_t* __restrict__ tokens) {
  const int32_t row = blockIdx.x * (kThreads / nvp::kWave) + threadIdx.x / nvp::kWave;
  if (row >= batch) return;
  const int lane = threadIdx.x & (nvp::kWave - 1);
  Best best{-INFINITY, INT32_MAX};
  for (int32_t c = lane; c < chunks; c += nvp::kWave)
    take(best, part_score[static_cast<int64_t>(row) * chunks + c],
         part_index[static_cast<int64_t>(row) * chunks + c]);
  best = wave_best(best);
  if (lane == 0) tokens[row] = best.i;
}

// Work split.  Batches of kRowPlanBatch rows or more: one wide workgroup per row
// (batch 256 x 151,936, flushed cache: 40.8 us against 41.8 for the best split; an
// all-greedy batch 13.8 against 20.6 us).  Smaller batches: enough workgroups to
// cover the chip many times over, each streaming at least kMinChunk elements, chunk
// lengths multiples of kUnit (batch 256 split into 2048 groups 45.3 us, 4096 42.8,
// 8192 41.8), and a merge kernel.
constexpr int64_t kTargetGroups = 8192;
constexpr int32_t kMinChunk = 4096;

struct Plan {
  int32_t chunk;
  int32_t chunks;
};

Plan plan_for(int32_t batch, int32_t vocab) {
  if (batch >= kRowPlanBatch) {
    const int64_t chunk = (static_cast<int64_t>(vocab) + kUnit - 1) / kUnit * kUnit;
    return Plan{static_cast<int32_t>(chunk), 1};
  }
  int64_t want = (kTargetGroups + batch - 1) / batch;
  const int64_t most = (static_cast<int64_t>(vocab) + kMinChunk - 1) / kMinChunk;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int64_t chunk = (vocab + want - 1) / want;
  chunk = (chunk + kUnit - 1) / kUnit * kUnit;
  const int64_t chunks = (vocab + chunk - 1) / chunk;
  return Plan{static_cast<int32_t>(chunk), static_cast<int32_t>(chunks)};
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <typename DT, bool VEC>
void launch_partial(const void* logits, int64_t ls, const float* temps, const float* gumbel,
                    int64_t gs, int32_t vocab, const Plan& p, int32_t batch, float* ps,
                    int32_t* pi, int32_t* tokens, hipStream_t s) {
  const auto* z = static_cast<const typename DT::T*>(logits);
  if (batch >= kRowPlanBatch)
    sample_partial_kernel<DT, VEC, kRowThreads, kRowUnroll>
        <<<dim3(p.chunks, batch), dim3(kRowThreads), 0, s>>>(z, ls, temps, gumbel, gs, vocab,
                                                             p.chunk, p.chunks, ps, pi, tokens);
  else
    sample_partial_kernel<DT, VEC, kThreads, kUnroll>
        <<<dim3(p.chunks, batch), dim3(kThreads), 0, s>>>(z, ls, temps, gumbel, gs, vocab,
                                                          p.chunk, p.chunks, ps, pi, tokens);
}

}  // namespace

extern "C" size_t nv_sample_workspace_size(int32_t batch, int32_t vocab) {
  if (batch <= 0 || vocab <= 0) return 0;
  const Plan p = plan_for(batch, vocab);
  if (p.chunks == 1) return 0;
  const size_t n = static_cast<size_t>(batch) * p.chunks;
  return align256(n * sizeof(float)) + align256(n * sizeof(int32_t));
}

extern "C" nv_status nv_sample(int32_t* tokens, const void* logits, int64_t logits_row_stride,
                               const float* temperatures, const float* gumbel,
                               int64_t gumbel_row_stride, int32_t batch, int32_t vocab,
                               int32_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (batch < 0 || vocab <= 0) return NV_ERR_INVALID_ARG;
  if (dtype != NV_F32 && dtype != NV_BF16) return NV_ERR_UNSUPPORTED;
  if (batch == 0) return NV_OK;
  if (batch > 65535 || vocab > 0x7fffff00) return NV_ERR_UNSUPPORTED;  // grid rows; int32 chunks
  if (!tokens || !logits || !temperatures || !gumbel) return NV_ERR_INVALID_ARG;
  if (logits_row_stride < vocab || gumbel_row_stride < vocab) return NV_ERR_INVALID_ARG;
  const Plan p = plan_for(batch, vocab);
  const size_t need = nv_sample_workspace_size(batch, vocab);
  if (workspace_bytes < need || (need > 0 && !workspace)) return NV_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 3)) return NV_ERR_INVALID_ARG;
  float* ps = nullptr;
  int32_t* pi = nullptr;
  if (need > 0) {
    const size_t n = static_cast<size_t>(batch) * p.chunks;
    ps = static_cast<float*>(workspace);
    pi = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align256(n * sizeof(float)));
  }
  if (nvp_check::on()) {
    const nv_status st = nvp_check::sample(temperatures, batch, stream);
    if (st != NV_OK) return st;
  }
  const int64_t esize = dtype == NV_F32 ? 4 : 2;
  const uintptr_t align = reinterpret_cast<uintptr_t>(logits) |
                          reinterpret_cast<uintptr_t>(gumbel) |
                          static_cast<uintptr_t>(logits_row_stride * esize) |
                          static_cast<uintptr_t>(gumbel_row_stride * 4);
  const bool vec = (align & 15) == 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == NV_BF16) {
    if (vec)
      launch_partial<nvp::BF16, true>(logits, logits_row_stride, temperatures, gumbel,
                                      gumbel_row_stride, vocab, p, batch, ps, pi, tokens, s);
    else
      launch_partial<nvp::BF16, false>(logits, logits_row_stride, temperatures, gumbel,
                                       gumbel_row_stride, vocab, p, batch, ps, pi, tokens, s);
  } else {
    if (vec)
      launch_partial<nvp::F32, true>(logits, logits_row_stride, temperatures, gumbel,
                                     gumbel_row_stride, vocab, p, batch, ps, pi, tokens, s);
    else
      launch_partial<nvp::F32, false>(logits, logits_row_stride, temperatures, gumbel,
                                      gumbel_row_stride, vocab, p, batch, ps, pi, tokens, s);
  }
  nv_status st = nvp_host::launch_status();
  if (st != NV_OK || p.chunks == 1) return st;
  const int rows_per_group = kThreads / nvp::kWave;
  sample_merge_kernel<<<dim3((batch + rows_per_group - 1) / rows_per_group), dim3(kThreads), 0,
                        s>>>(ps, pi, p.chunks, batch, tokens);
  return nvp_host::launch_status();
}
