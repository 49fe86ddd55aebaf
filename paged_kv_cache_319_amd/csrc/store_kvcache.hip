// store_kvcache: scatter this step's new K/V rows into the paged cache by slot.
//
// Walkthrough (xingyun3d.csdn.net nano-vllm article), section 七: before
// attention a lightweight kernel writes the step's K/V into the pre-allocated
// cache at slot_mapping; the gitcode.csdn.net summary (section 三.4) describes
// it as a plain copy.  Here each thread moves one VEC-byte piece of a K row and
// the same piece of the V row; a row (num_kv_heads * head_dim elements) is
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

template <int VEC>
__global__ __launch_bounds__(256) void store_kvcache_kernel(
    const char* __restrict__ k, const char* __restrict__ v, int64_t k_stride, int64_t v_stride,
    char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t pieces_per_row,
    int64_t row_bytes) {
  using V = typename VecT<VEC>::T;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = gid / pieces_per_row;
  if (row >= num_tokens) return;
  const int64_t piece = gid - row * pieces_per_row;
  const int32_t slot = slot_mapping[row];
  if (slot < 0) return;
  const int64_t off = piece * VEC;
  const V kv = *reinterpret_cast<const V*>(k + row * k_stride + off);
  const V vv = *reinterpret_cast<const V*>(v + row * v_stride + off);
  const int64_t dst = static_cast<int64_t>(slot) * row_bytes + off;
  *reinterpret_cast<V*>(k_cache + dst) = kv;
  *reinterpret_cast<V*>(v_cache + dst) = vv;
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
  const int block = 256;
  const int64_t grid = (threads + block - 1) / block;
  if (grid > 0x7fffffff) return NV_ERR_INVALID_ARG;
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
    case 16:
      store_kvcache_kernel<16><<<dim3(grid), dim3(block), 0, s>>>(
          kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, static_cast<int32_t>(pieces), row_bytes);
      break;
    case 8:
      store_kvcache_kernel<8><<<dim3(grid), dim3(block), 0, s>>>(
          kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, static_cast<int32_t>(pieces), row_bytes);
      break;
    case 4:
      store_kvcache_kernel<4><<<dim3(grid), dim3(block), 0, s>>>(
          kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, static_cast<int32_t>(pieces), row_bytes);
      break;
    default:
      store_kvcache_kernel<2><<<dim3(grid), dim3(block), 0, s>>>(
          kc, vc, ks, vs, kd, vd, slot_mapping, num_tokens, static_cast<int32_t>(pieces), row_bytes);
      break;
  }
  return nvp_host::launch_status();
}
