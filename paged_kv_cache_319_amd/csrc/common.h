// Shared device helpers for the nvpaged kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvpaged.h"

namespace nvp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Element traits: storage type and how many elements one 16-byte lane load holds.
struct F32 {
  using T = float;
  static constexpr int kBytes = 4;
  static constexpr int kPerLoad = 4;
};
struct BF16 {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kPerLoad = 8;
};

// bfloat16 <-> float.  A bfloat16 is the high half of a binary32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Widen one 16-byte lane load to floats.
template <typename DT>
__device__ __forceinline__ void widen(const u32x4& r, float* x);

template <>
__device__ __forceinline__ void widen<F32>(const u32x4& r, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r[i]);
}

template <>
__device__ __forceinline__ void widen<BF16>(const u32x4& r, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(r[i]);
    x[2 * i + 1] = bf16_hi(r[i]);
  }
}

// Dot product of two 16-byte lane loads, accumulated in fp32.
template <typename DT>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float acc);

template <>
__device__ __forceinline__ float dot16<F32>(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
  return acc;
}

template <>
__device__ __forceinline__ float dot16<BF16>(const u32x4& a, const u32x4& b, float acc) {
  // bf16 x bf16 products are exact in fp32; v_dot2 adds two of them per step.
  // Vector elements are copied to scalars before the bit cast: a bit cast applied
  // directly to an element of an ext_vector_type reads element 0 with this compiler.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ai = a[i], bi = b[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ai),
                                          __builtin_bit_cast(bf16x2_t, bi), acc, false);
  }
  return acc;
}

// Cross-lane moves.  DPP row operations stay inside 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

constexpr int kDppXor1 = 0xb1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

// Sum over aligned groups of N consecutive lanes (N in 1..64, power of two);
// every lane of a group receives the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16, kWave));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32, kWave));
  return x;
}

// Sum over lanes that are STRIDE apart (STRIDE a power of two, STRIDE..32):
// folds the 64 / STRIDE lanes sharing lane % STRIDE.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
#pragma unroll
  for (int s = STRIDE; s < kWave; s *= 2) x += __shfl_xor(x, s, kWave);
  return x;
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <typename DT>
__device__ __forceinline__ void store_out(typename DT::T* p, float v);

template <>
__device__ __forceinline__ void store_out<F32>(float* p, float v) { *p = v; }

template <>
__device__ __forceinline__ void store_out<BF16>(uint16_t* p, float v) {
  *p = static_cast<uint16_t>(f32_to_bf16_rne(v));
}

}  // namespace nvp

// Host-side helpers shared by the entry points.
namespace nvp_host {

inline nv_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NV_OK : NV_ERR_HIP;
}

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace nvp_host

// Check mode (check.hip): validation of the device-data preconditions before a launch.
namespace nvp_check {
bool on();
nv_status store(const int32_t* slots, int32_t n, int32_t num_blocks, int32_t block_size,
                void* stream);
nv_status decode(const int32_t* tables, int32_t width, const int32_t* lens,
                 const int32_t* schedule, const int32_t* new_slots, int32_t batch,
                 int32_t block_size, int32_t num_blocks, int32_t max_len, void* stream);
nv_status prefill(const int32_t* cu_q, const int32_t* cu_k, const int32_t* tables, int32_t width,
                  int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t max_q,
                  int32_t max_k, const int32_t* tiles, int32_t num_tiles, int32_t tile_rows,
                  void* stream);
nv_status sample(const float* temperatures, int32_t batch, void* stream);
}  // namespace nvp_check
