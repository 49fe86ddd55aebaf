// store_kvcache: scatter this step's new K/V rows into the paged cache by slot.
//
// Walkthrough (xingyun3d.csdn.net nano-vllm article), section 七: before
// attention a lightweight kernel writes the step's K/V into the pre-allocated
// cache at slot_mapping; the gitcode.csdn.net summary (section 三.4) describes
// it as a plain copy.  Here each thread moves one or two VEC-byte pieces of K rows
// and the same pieces of the V rows; a row (num_kv_heads * head_dim elements) is
// contiguous both in the source and in the cache, so every wave issues fully
// coalesced loads and stores.  Rows whose slot is -1 are skipped.  The copy
// moves raw bits, so it is exact for any payload, NaN included.
#include "common.h"

namespace {

template <int VEC>
struct VecT;
template <>
struct VecT<16> { using T = nvp::u32x4; };
template <>
struct VecT<8> { using T = uint2; };
template <>
struct VecT<4> { using T = uint32_t; };
template <>
struct VecT<2> { using T = uint16_t; };

constexpr int kThreads = 256;

// A workgroup moves PER * 256 consecutive pieces; thread t takes pieces t, t + 256, ...
// of that span and issues all its loads before its stores (16-byte pieces: PER = 2,
// measured 8.7 vs 9.3 us for the 6 650-row prefill store; PER = 4 was slower).
template <int VEC, int PER>
__global__ __launch_bounds__(kThreads) void store_kvcache_kernel(
    const char* __restrict__ k, const char* __restrict__ v, int64_t k_stride, int64_t v_stride,
    char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t pieces_per_row,
    int64_t row_bytes) {
  using V = typename VecT<VEC>::T;
  const int64_t total = static_cast<int64_t>(num_tokens) * pieces_per_row;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kThreads * PER + threadIdx.x;
  V kv[PER], vv[PER];
  int64_t dst[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int64_t gid = first + p * kThreads;
    dst[p] = -1;
    if (gid >= total) continue;
    const int64_t row = gid / pieces_per_row;
    const int32_t slot = slot_mapping[row];
    if (slot < 0) continue;
    const int64_t off = (gid - row * pieces_per_row) * VEC;
    kv[p] = *reinterpret_cast<const V*>(k + row * k_stride + off);
    vv[p] = *reinterpret_cast<const V*>(v + row * v_stride + off);
    dst[p] = static_cast<int64_t>(slot) * row_bytes + off;
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    if (dst[p] < 0) continue;
    *reinterpret_cast<V*>(k_cache + dst[p]) = kv[p];
    *reinterpret_cast<V*>(v_cache + dst[p]) = vv[p];
  }
}

template <int VEC, int PER>
void launch_store(const char* kc, const char* vc, int64_t ks, int64_t vs, char* kd, char* vd,
                  const int32_t* slots, int32_t num_tokens, int64_t pieces, int64_t row_bytes,
                  hipStream_t s) {
  const int64_t grid = (pieces * num_tokens + kThreads * PER - 1) / (kThreads * PER);
  store_kvcache_kernel<VEC, PER><<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s>>>(
      kc, vc, ks, vs, kd, vd, slots, num_tokens, static_cast<int32_t>(pieces), row_bytes);
}

int pick_vec(uintptr_t bits) {
  if ((bits & 15) == 0) return 16;
  if ((bits & 7) == 0) return 8;
  if ((bits & 3) == 0) return 4;
  return 2;
}

}  // namespace

extern "C" nv_status nv_store_kvcache(const void* k, const void* v, int64_t k_row_stride,
                                      int64_t v_row_stride, void* k_cache, void* v_cache,
                                      const int32_t* slot_mapping, int32_t num_tokens,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t num_blocks, int32_t block_size, int32_t dtype,
                                      void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
      block_size <= 0)
    return NV_ERR_INVALID_ARG;
  if (dtype != NV_F32 && dtype != NV_BF16) return NV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return NV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return NV_ERR_INVALID_ARG;
  const int64_t esize = dtype == NV_F32 ? 4 : 2;
  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * esize;
  if (k_row_stride < static_cast<int64_t>(num_kv_heads) * head_dim ||
      v_row_stride < static_cast<int64_t>(num_kv_heads) * head_dim)
    return NV_ERR_INVALID_ARG;
  const int64_t ks = k_row_stride * esize, vs = v_row_stride * esize;
  const uintptr_t align = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                          reinterpret_cast<uintptr_t>(k_cache) |
                          reinterpret_cast<uintptr_t>(v_cache) | static_cast<uintptr_t>(ks) |
                          static_cast<uintptr_t>(vs) | static_cast<uintptr_t>(row_bytes);
  const int vec = pick_vec(align);
  const int64_t pieces = row_bytes / vec;
  const int64_t threads = pieces * num_tokens;
  if ((threads + kThreads - 1) / kThreads > 0x7fffffff) return NV_ERR_INVALID_ARG;
  if (nvp_check::on()) {
    const nv_status st = nvp_check::store(slot_mapping, num_tokens, num_blocks, block_size, stream);
    if (st != NV_OK) return st;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* kc = static_cast<const char*>(k);
  const char* vc = static_cast<const char*>(v);
  char* kd = static_cast<char*>(k_cache);
  char* vd = static_cast<char*>(v_cache);
  switch (vec) {
    case 16: launch_store<16, 2>(kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, pieces, row_bytes, s); break;
    case 8: launch_store<8, 1>(kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, pieces, row_bytes, s); break;
    case 4: launch_store<4, 1>(kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, pieces, row_bytes, s); break;
    default: launch_store<2, 1>(kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, pieces, row_bytes, s); break;
  }
  return nvp_host::launch_status();
}
