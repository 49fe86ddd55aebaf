// Packed varlen causal prefill attention over a paged KV cache, on MFMA.
//
// Operation (walkthrough, xingyun3d.csdn.net nano-vllm article, sections 七 and
// 八): the prefill call takes the packed queries of the uncached tokens, the
// cache, cu_seqlens_q / cu_seqlens_k and the block table; every key, cached
// prefix and new token alike, is read from the cache through the block table.
// Query row i of sequence s is the token at position k_s - n_s + i and, with
// the causal mask, attends keys 0 .. k_s - n_s + i.  Scores are
// softmax(Q K^T / sqrt(d)) V ("万字深度解析 Nano-vLLM", section 1.2); query head h
// reads KV head h / g (same article, section 3.2.1).
//
// Tiling.  A workgroup of eight waves owns 32 * PB query positions of one
// sequence and GW query heads that share one KV head (GW * PB = 8): wave w takes
// head w % GW and position block w / GW.  K/V are walked in tiles of BN keys;
// each tile is gathered through the block table once per workgroup into LDS
// (K row-major; V row-major and read transposed for bf16, transposed on its way
// in for fp32) and serves all eight waves.  Two LDS buffers let
// the next tile's global loads and LDS writes overlap this tile's MFMA work with
// one barrier per tile; two waves per SIMD hide each other's softmax and LDS
// latency.  A wave skips tiles that its causal rows cannot see and masks only
// the tiles that cross its diagonal.  bf16 output rows are written through the
// then idle tile buffers so that every store covers whole rows.
//
// Per wave and tile, with v_mfma_f32_32x32x16_bf16 (eight v_mfma_f32_32x32x2f32
// for fp32 data):
//   S^T[key, query] = K Q^T     -- A = K rows from LDS, B = Q held in registers;
//   online softmax per query column: the accumulator layout gives each lane one
//   query and 16 of the keys of a 32-key block, the other 16 sit in lane ^ 32,
//   so the row maximum costs one cross-lane exchange;
//   O^T[d, query] += V^T P^T    -- B = P^T straight from the S^T registers,
//   A = V^T from the transposed LDS tile, with the key order matched to the
//   order in which the S^T accumulator holds the keys.
// The contraction index of an MFMA may be permuted freely as long as A and B
// agree, which is what lets P^T feed the second product without a shuffle.
#include <type_traits>

#include "common.h"

namespace {

using namespace nvp;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Eight contraction elements of one MFMA operand held by one lane.
template <typename DT>
struct Frag;
template <>
struct Frag<BF16> {
  u32x4 v;
};
template <>
struct Frag<F32> {
  u32x4 v[2];
};

__device__ __forceinline__ f32x16 mma(const Frag<BF16>& a, const Frag<BF16>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                 __builtin_bit_cast(bf16x8_t, b.v), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mma(const Frag<F32>& a, const Frag<F32>& b, f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t ae = a.v[e / 4][e % 4], be = b.v[e / 4][e % 4];
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ae), __uint_as_float(be), c, 0, 0, 0);
  }
  return c;
}

// Eight contiguous elements (a row slice) from memory into a fragment.
template <typename DT>
__device__ __forceinline__ void frag_load(Frag<DT>& f, const typename DT::T* p);
template <>
__device__ __forceinline__ void frag_load<BF16>(Frag<BF16>& f, const uint16_t* p) {
  f.v = *reinterpret_cast<const u32x4*>(p);
}
template <>
__device__ __forceinline__ void frag_load<F32>(Frag<F32>& f, const float* p) {
  f.v[0] = *reinterpret_cast<const u32x4*>(p);
  f.v[1] = *reinterpret_cast<const u32x4*>(p + 4);
}

template <typename DT>
__device__ __forceinline__ void frag_negate(Frag<DT>& f);
template <>
__device__ __forceinline__ void frag_negate<BF16>(Frag<BF16>& f) {
  f.v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
}
template <>
__device__ __forceinline__ void frag_negate<F32>(Frag<F32>& f) {
  f.v[0] ^= u32x4{0x80000000u, 0x80000000u, 0x80000000u, 0x80000000u};
  f.v[1] ^= u32x4{0x80000000u, 0x80000000u, 0x80000000u, 0x80000000u};
}

template <typename DT>
__device__ __forceinline__ void frag_zero(Frag<DT>& f);
template <>
__device__ __forceinline__ void frag_zero<BF16>(Frag<BF16>& f) { f.v = u32x4{0, 0, 0, 0}; }
template <>
__device__ __forceinline__ void frag_zero<F32>(Frag<F32>& f) {
  f.v[0] = u32x4{0, 0, 0, 0};
  f.v[1] = u32x4{0, 0, 0, 0};
}

// Two runs of four consecutive elements (p0[0..3], p1[0..3]) into a fragment.
template <typename DT>
__device__ __forceinline__ void frag_load_2x4(Frag<DT>& f, const typename DT::T* p0,
                                              const typename DT::T* p1);
template <>
__device__ __forceinline__ void frag_load_2x4<F32>(Frag<F32>& f, const float* p0, const float* p1) {
  f.v[0] = *reinterpret_cast<const u32x4*>(p0);
  f.v[1] = *reinterpret_cast<const u32x4*>(p1);
}

// Softmax weights (fp32) -> fragment of the data type.  Two values convert in one
// v_cvt_pk_bf16_f32 (round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <typename DT>
__device__ __forceinline__ void frag_from_f32(Frag<DT>& f, const float* x);
template <>
__device__ __forceinline__ void frag_from_f32<BF16>(Frag<BF16>& f, const float* x) {
  f.v = u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
              pack_bf16(x[6], x[7])};
}
template <>
__device__ __forceinline__ void frag_from_f32<F32>(Frag<F32>& f, const float* x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e / 4][e % 4] = __float_as_uint(x[e]);
}

// Two transposing 8-byte LDS reads (ds_read_b64_tr_b16) into one bf16 fragment.  Within
// each group of 16 lanes, lane i receives element i % 4 of the pieces that lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 point at.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
__device__ __forceinline__ u32x4 tr_pair(const uint16_t* p0, const uint16_t* p1) {
  // p0, p1 point into __shared__ memory: the casts are generic -> LDS address space.
  const auto a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p0));
  const auto b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p1));
  const uint2 ua = __builtin_bit_cast(uint2, a);
  const uint2 ub = __builtin_bit_cast(uint2, b);
  return u32x4{ua.x, ua.y, ub.x, ub.y};
}

// Four output elements (consecutive head_dim positions) -> memory.
template <typename DT>
__device__ __forceinline__ void store4(typename DT::T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<BF16>(uint16_t* p, float a, float b, float c, float d) {
  // v_cvt_pk_bf16_f32 rounds to nearest even, as the output rounding requires
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(a, b), pack_bf16(c, d));
}
template <>
__device__ __forceinline__ void store4<F32>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Transpose four 16-byte key-row slices (keys x0..x3, EPC elements each) into EPC
// runs of four keys and write them to the transposed V tile.
template <typename DT>
__device__ __forceinline__ void write_vt(typename DT::T* vt, int vrow, int d0, int k0,
                                         const u32x4* r);
template <>
__device__ __forceinline__ void write_vt<F32>(float* vt, int vrow, int d0, int k0, const u32x4* r) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
    *reinterpret_cast<u32x4*>(vt + (d0 + m) * vrow + k0) = u32x4{r[0][m], r[1][m], r[2][m], r[3][m]};
}

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_tables;
  const int32_t* tile_schedule;  // (sequence, query tile) pairs, heaviest first; or null
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t group;
  int32_t causal;
  int32_t bs_shift;    // log2(block_size) when it is a power of two, else -1
  int32_t negate_q;    // the softmax scale is negative: q is negated, scale_log2 > 0
  float scale_log2;    // |softmax_scale| * log2(e), > 0
};

// BMODE: how a staging wave finds the cache block of its keys: 1 for a power-of-two block
// size (shift and mask), 0 for any other multiple of 16 (division).
// Lanes l and l ^ 32 combined without LDS: v_permlane32_swap of a value with itself
// swaps the upper half of one copy with the lower half of the other, so in every lane the
// two results hold the lane's own value and its partner's (a maximum or a sum of the pair
// then needs no cross-lane read through LDS and no wait on the LDS counter).
__device__ __forceinline__ void halves32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __uint_as_float(r0);
  b = __uint_as_float(r1);
}

template <typename DT, int D, int GW, int PB, int BN, int BMODE>
__global__ __launch_bounds__(64 * GW * PB) void paged_prefill_kernel(PrefillArgs a) {
  using T = typename DT::T;
  constexpr int ES = DT::kBytes;
  constexpr int EPC = 16 / ES;           // elements per 16-byte chunk
  constexpr int CPR = D / EPC;           // chunks per key row
  constexpr int KSTEPS = D / 16;         // contraction steps over head_dim
  constexpr int DT32 = D / 32;           // 32-row output tiles over head_dim
  constexpr int NKB = BN / 32;           // 32-key blocks per tile
  constexpr int NKS = BN / 16;           // 16-key contraction slices per tile
  constexpr int KROW = D + EPC;          // padded K row (elements)
  // bf16: V is kept row-major in LDS and read transposed (ds_read_b64_tr_b16); its rows
  // are padded to 32 elements past head_dim.  The LDS serves 32 lanes of such a read at
  // once over 64 banks of 4 bytes; those lanes cover 4 rows x 64 bytes, and a row stride
  // of 16 (mod 64) banks puts the four rows in disjoint banks (the hardware's bank-
  // conflict counter reads 0; 16 elements of padding gave a 2-way conflict).  fp32: V is
  // transposed on the way into LDS, rows of BN + 4 keys.
  constexpr bool TRV = DT::kBytes == 2;
  constexpr int VROW = TRV ? D + 32 : BN + 4;
  constexpr int VBUF = TRV ? BN * VROW : D * VROW;
  constexpr int UNITS = (BN / 4) * CPR;  // 4-key x 16-byte staging units per tile
  constexpr int NT = 64 * GW * PB;       // threads per workgroup
  constexpr int HALF = NT / 2;           // the first half stages K, the second V
  constexpr int BMW = 32 * PB;           // query positions per workgroup

  // Two K / V^T tile buffers: the next tile is written while this one is read.
  __shared__ __attribute__((aligned(16))) T ks[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) T vt[2][VBUF];

  // Work tile: from the host schedule (grid = heads x tiles, heaviest tiles first), or
  // the dense grid (tiles x heads x sequences, a sequence's late tiles first).
  int s, qt, hy;
  if (a.tile_schedule) {
    hy = blockIdx.x;
    s = a.tile_schedule[2 * blockIdx.y];
    qt = a.tile_schedule[2 * blockIdx.y + 1];
  } else {
    hy = blockIdx.y;
    s = blockIdx.z;
    qt = gridDim.x - 1 - blockIdx.x;
  }
  const int q_begin = a.cu_q[s];
  const int n = a.cu_q[s + 1] - q_begin;
  const int wg_q0 = qt * BMW;
  if (wg_q0 >= n) return;                      // uniform over the workgroup
  const int k_len = a.cu_k[s + 1] - a.cu_k[s];
  const int p0 = k_len - n;                    // cached prefix length

  const int subgroups = a.group / GW;
  const int j = hy / subgroups;
  const int sub = hy % subgroups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int head = j * a.group + sub * GW + (wave % GW);
  const int q0 = wg_q0 + (wave / GW) * 32;     // first query row of this wave
  const int qi = lane & 31;                    // query column held by this lane
  const int hh = lane >> 5;                    // contraction half held by this lane

  const int k_end = a.causal ? p0 + min(wg_q0 + BMW, n) : k_len;  // keys any row can see
  const int ntiles = (k_end + BN - 1) / BN;

  const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
  const int32_t* __restrict__ bt = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  // The table does not change while the kernel runs: read through the constant address
  // space, its workgroup-uniform entries become scalar loads (no wait on vector memory).
  typedef const __attribute__((address_space(4))) int32_t cint32_t;
  const cint32_t* btc = (const cint32_t*)(bt);
  const int64_t slot_stride = static_cast<int64_t>(a.num_kv_heads) * D;

  // Q^T operand: query row q0 + qi, head_dim elements 16*kk + 8*hh + 0..7.  Rows past
  // the sequence read its first row and are zeroed; the loads complete here, before the
  // tile loop (the zeroing select consumes them), so no wait inside the loop is left
  // pending on them.
  Frag<DT> qf[KSTEPS];
  {
    const bool qv = q0 + qi < n;
    const int qrow = q_begin + (qv ? q0 + qi : 0);
    const T* qp = static_cast<const T*>(a.q) +
                  (static_cast<int64_t>(qrow) * a.num_q_heads + head) * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) frag_load<DT>(qf[kk], qp + 16 * kk);
    // A negative scale is applied as |scale| to -q (a sign flip, exact).
    const bool neg = a.negate_q != 0;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (neg) frag_negate<DT>(qf[kk]);
      if (!qv) frag_zero<DT>(qf[kk]);
    }
  }

  // Staging: the first half of the workgroup's waves stages K, the second half V.  Each
  // of a role's four waves gathers KPW consecutive keys of a tile, one unit (4 keys x one
  // 16-byte chunk) per lane; lanes past UPW hold none.  A wave's keys start at a multiple
  // of KPW, which divides 16, so they lie in one cache block for every block size (a
  // multiple of 16): one wave-uniform table load per wave and tile (a scalar load,
  // which never waits on the vector loads in flight), and the wave's loads are buffer
  // loads through a resource whose range ends at k_end.  The hardware range check
  // returns zeros for keys at or past k_end, so a tile's tail needs no selects on the
  // load side and no zeroing on the LDS side (V must be finite there: its weight is 0).
  static_assert(HALF == 256 && UNITS % 4 == 0 && UNITS / 4 <= 64, "four staging waves");
  constexpr int UPW = UNITS / 4;          // units per staging wave
  constexpr int KPW = 4 * UPW / CPR;      // keys per staging wave (16 bf16, 8 fp32)
  static_assert(4 * KPW == BN && 16 % KPW == 0, "a staging wave's keys lie in one block");
  const bool v_role = wave >= (GW * PB) / 2;   // wave-uniform
  const int rtid = tid - (v_role ? HALF : 0);
  const int swave = v_role ? wave - (GW * PB) / 2 : wave;   // staging wave in the role (uniform)
  const bool s_on = (rtid & 63) < UPW;         // this lane holds a unit
  const int my_unit = swave * UPW + (rtid & 63);
  const int my_c = my_unit % CPR;              // the unit's 16-byte chunk of a row
  const int my_kg = my_unit / CPR;             // the unit's first key is 4 * my_kg
  const T* __restrict__ src = v_role ? vc : kc;
  u32x4 stA[4];
  const int last_entry = a.max_blocks - 1;
  const uint32_t row_bytes = static_cast<uint32_t>(slot_stride) * ES;
  uint32_t voff[4];   // byte offsets of the lane's pieces from the wave's first key
#pragma unroll
  for (int x = 0; x < 4; ++x)
    voff[x] = (4 * my_kg + x - KPW * swave) * row_bytes + my_c * 16;
  auto load_tile = [&](int tile, u32x4 (&st)[4]) {
    const int kw0 = tile * BN + KPW * swave;   // the wave's first key
    int blk = 0, off = 0;
    if (kw0 < k_end) {
      if constexpr (BMODE != 0) {
        blk = btc[min(kw0 >> a.bs_shift, last_entry)];
        off = kw0 & ((1 << a.bs_shift) - 1);
      } else {
        const int lb = min(kw0 / a.block_size, last_entry);
        blk = btc[lb];
        off = kw0 - lb * a.block_size;
      }
    }
    const T* __restrict__ base =
        src + (static_cast<int64_t>(blk) * a.block_size + off) * slot_stride +
        static_cast<int64_t>(j) * D;
    const int valid = min(max(k_end - kw0, 0), KPW);
    // every input is wave-uniform; readfirstlane lets the compiler see it (readfirstlane
    // returns int: each half goes back through uint32_t before it is widened, or a low
    // word with bit 31 set would sign-extend into the high word).  Resource word 3
    // (0x00020000): 32-bit data format, so the untyped 16-byte loads are range-checked
    // against nrec bytes (stride 0: raw offsets).
    const uint64_t b64 = reinterpret_cast<uint64_t>(base);
    const uint32_t b_hi = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b64 >> 32))));
    const uint32_t b_lo = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b64))));
    const uint64_t bu = (static_cast<uint64_t>(b_hi) << 32) | static_cast<uint64_t>(b_lo);
    const int nrec = __builtin_amdgcn_readfirstlane(static_cast<int>(valid * row_bytes));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(bu), static_cast<short>(0), nrec, 0x00020000);
    if (s_on) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        st[x] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, static_cast<int>(voff[x]), 0, 0));
    }
  };
  // LDS write of a staged tile: K rows as they are; V rows as they are (bf16) or
  // transposed (fp32).
  auto store_tile = [&](T* buf, const u32x4 (&st)[4]) {
    if (!s_on) return;
    if (!v_role) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        *reinterpret_cast<u32x4*>(&buf[(4 * my_kg + x) * KROW + my_c * EPC]) = st[x];
    } else if constexpr (TRV) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        *reinterpret_cast<u32x4*>(&buf[(4 * my_kg + x) * VROW + my_c * EPC]) = st[x];
    } else {
      write_vt<DT>(buf, VROW, my_c * EPC, 4 * my_kg, st);
    }
  };

  f32x16 oacc[DT32];
#pragma unroll
  for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY;   // running max of this lane's query (log2 domain)
  float l_run = 0.f;         // running sum over this lane's half of the keys

  const int qpos = p0 + q0 + qi;                        // absolute position of the query
  const int key_limit = a.causal ? min(qpos + 1, k_len) : k_len;
  // Per wave: keys visible to every query row (no mask below this), keys visible to
  // any row, and the number of tiles the wave computes.
  const int all_see = a.causal ? min(p0 + q0 + 1, k_len) : k_len;
  const int any_sees = a.causal ? p0 + min(q0 + 32, n) : k_len;
  const int wtiles = q0 < n ? min(ntiles, (any_sees + BN - 1) / BN) : 0;

  // S^T = K Q^T for the 32-key blocks of one tile; the blocks' accumulation chains are
  // interleaved so consecutive MFMAs are independent.
  auto qk = [&](const T* kl, f32x16 (&sacc)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        Frag<DT> kf;
        frag_load<DT>(kf, &kl[(32 * kb + qi) * KROW + 16 * kk + 8 * hh]);
        sacc[kb] = mma(kf, qf[kk], sacc[kb]);
      }
    }
  };

  // Online softmax, first half: mask (on tiles that cross the wave's diagonal) and the
  // tile maximum.  Register r of block kb holds key 32*kb + 8*(r/4) + 4*hh + r%4 of the
  // tile for query column qi; its partner lane (lane ^ 32) holds the other half of the
  // keys, so the maximum costs one exchange.  The running maximum only moves when a
  // tile exceeds it by more than 2^8 (weights then stay at most 256 and the rescale of
  // O is rare); O and l always share one reference, so the softmax is unchanged.
  // Returns the reference for the exponents; alpha is the rescale factor of O and l.
  auto tile_max = [&](auto mask_c, int tile, f32x16 (&sacc)[NKB], float& alpha) {
    constexpr bool MASK = decltype(mask_c)::value;
    // key = tile*BN + 32*kb + 8*(r/4) + 4*hh + r%4 is visible iff key < key_limit
    const int lim = key_limit - tile * BN - 4 * hh;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (MASK)
          sacc[kb][r] = 32 * kb + 8 * (r / 4) + (r % 4) < lim ? sacc[kb][r] : -INFINITY;
        tmax = fmaxf(tmax, sacc[kb][r]);
      }
    {
      float a0, a1;
      halves32(tmax, a0, a1);
      tmax = fmaxf(a0, a1);
    }
    const float m_tile = tmax == -INFINITY ? -INFINITY : tmax * a.scale_log2;
    const float m_use = m_tile > m_run + 8.f ? m_tile : m_run;
    const float m_ref = m_use == -INFINITY ? 0.f : m_use;
    alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    m_run = m_use;
    return m_ref;
  };

  // Second half, fused with O^T += V^T P^T one 32-key block at a time: weights
  // 2^(s*scale_log2 - m) (the scale, > 0, applied by one fma per score), their sum, the
  // bf16 (or fp32) fragments, and the MFMAs over the block's two 16-key slices.
  // Fragment element e of slice ks holds key 16*ks + 8*(e/4) + 4*hh + e%4, matching the
  // S^T register order.  The head_dim tiles are the inner loop: their accumulators are
  // independent.
  const int tr_off = (4 * hh + ((lane & 15) >> 2)) * VROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto softmax_pv = [&](const T* vl, const f32x16 (&sacc)[NKB], float m_ref) {
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], a.scale_log2, -m_ref));
        psum += p[r];
      }
      Frag<DT> pf[2];
      frag_from_f32<DT>(pf[0], p);
      frag_from_f32<DT>(pf[1], p + 8);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int ksl = 2 * kb + h2;
#pragma unroll
        for (int dt = 0; dt < DT32; ++dt) {
          Frag<DT> vf;
          if constexpr (TRV) {
            // Transposed reads: lane l gets V[key0 + 0..3][32*dt + l%32], key0 = 16*ksl
            // + 4*hh (+ 8 for elements 4..7); each lane points its read at row key0 +
            // (l%16)/4, columns 32*dt + 16*((l/16)%2) + 4*(l%4) .. +3.
            const T* vb = vl + tr_off + (16 * ksl) * VROW + 32 * dt;
            vf.v = tr_pair(vb, vb + 8 * VROW);
          } else {
            const T* vrow = &vl[(32 * dt + qi) * VROW];
            frag_load_2x4<DT>(vf, vrow + 16 * ksl + 4 * hh, vrow + 16 * ksl + 8 + 4 * hh);
          }
          oacc[dt] = mma(vf, pf[h2], oacc[dt]);
        }
      }
    }
    l_run += psum;
  };

  // One tile step of a wave: the maximum of tile t's scores (in scur), the rare rescale
  // of O, then one straight-line block with S of tile t + 1 (K from kl, into snext) and
  // tile t's weights and P V (V from vl): the matrix cores and the vector ALUs work on
  // independent data.
  auto step = [&](int t, f32x16 (&scur)[NKB], f32x16 (&snext)[NKB], const T* kl,
                  const T* vl) {
    if (t >= wtiles) return;                       // wave-uniform
    float alpha;
    const float m_ref = (t + 1) * BN > all_see ? tile_max(std::true_type{}, t, scur, alpha)
                                               : tile_max(std::false_type{}, t, scur, alpha);
    l_run *= alpha;
    if (t > 0 && __builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {   // O is 0 before tile 0
#pragma unroll
      for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    // On the wave's last tile this S is not needed; computing it anyway (from whatever
    // finite values the buffer holds) keeps the block free of branches.
    qk(kl, snext);
    softmax_pv(vl, scur, m_ref);
    if constexpr (TRV) {
      // Schedule of the block (bf16): six LDS reads ahead, then per S MFMA one K read
      // and four vector instructions, per P V MFMA two V reads and three vector
      // instructions, so LDS latency and the softmax arithmetic hide under the MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // DS read
#pragma unroll
      for (int i = 0; i < NKB * KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0); // VALU
      }
#pragma unroll
      for (int i = 0; i < NKS * DT32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    }
  };

  // Tile pipeline.  In step t every wave reads K(t + 1) and V(t) from LDS; the K waves
  // write K(t + 2) and the V waves V(t + 1) into the other buffers (the ones read in
  // step t - 1), then issue the global loads of the tile they write in step t + 1, so
  // each load has a whole step to arrive.  One barrier per step.
  if (!v_role) {
    // The K waves fill two buffers before the first barrier: a second staging set,
    // live only here, puts tiles 0 and 1 in flight together (one memory latency at
    // the start of the workgroup instead of two).
    u32x4 stB[4];
    load_tile(0, stA);
    load_tile(1, stB);
    store_tile(ks[0], stA);
    load_tile(2, stA);
    store_tile(ks[1], stB);
  } else {
    load_tile(0, stA);
    store_tile(vt[0], stA);
    load_tile(1, stA);
  }
  __syncthreads();
  f32x16 sA[NKB], sB[NKB];
  if (wtiles > 0) qk(ks[0], sA);
  __syncthreads();                                 // K(0) is overwritten in step 0
  for (int t = 0; t < ntiles; t += 2) {
    if (!v_role) {
      store_tile(ks[0], stA);
      load_tile(t + 3, stA);
    } else {
      store_tile(vt[1], stA);
      load_tile(t + 2, stA);
    }
    step(t, sA, sB, ks[1], vt[0]);
    __syncthreads();
    if (t + 1 >= ntiles) break;
    if (!v_role) {
      store_tile(ks[1], stA);
      load_tile(t + 4, stA);
    } else {
      store_tile(vt[0], stA);
      load_tile(t + 3, stA);
    }
    step(t + 1, sB, sA, ks[0], vt[1]);
    __syncthreads();
  }

  // Normalise and write.  O^T register r of tile dt is head_dim position
  // 32*dt + 8*(r/4) + 4*hh + r%4 of query q0 + qi.
  float l_a, l_b;
  halves32(l_run, l_a, l_b);
  const float l_tot = l_a + l_b;
  if constexpr (TRV) {
    // bf16 rows leave through LDS: written straight from the registers, each store
    // instruction would cover 32 rows with 16 bytes apiece; read back row-major, it
    // covers OROWS whole rows.  The tile buffers are free after the last barrier: waves
    // 0-3 use K's, waves 4-7 V's, 32 rows each.  16-byte chunk c of row r sits at
    // position c ^ (r % OCH), so neither the writes nor the reads conflict in the banks.
    constexpr int OCH = D * DT::kBytes / 16;  // 16-byte chunks per row
    constexpr int OROWS = 64 / OCH;           // rows per store instruction
    static_assert(GW * PB == 8 && 4 * 32 * D <= 2 * BN * KROW && 4 * 32 * D <= 2 * VBUF,
                  "output staging fits the tile buffers");
    T* ob = (wave < 4 ? &ks[0][0] : &vt[0][0]) + (wave % 4) * 32 * D;
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int pos = (4 * dt + g4) ^ (qi % OCH);
        store4<DT>(ob + qi * D + pos * EPC + 4 * hh, oacc[dt][4 * g4] * inv,
                   oacc[dt][4 * g4 + 1] * inv, oacc[dt][4 * g4 + 2] * inv,
                   oacc[dt][4 * g4 + 3] * inv);
      }
    // Only this wave's rows: its own LDS writes complete in order, no barrier needed.
#pragma unroll
    for (int i = 0; i < 32 / OROWS; ++i) {
      const int r = i * OROWS + lane / OCH;
      const int pos = lane % OCH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&ob[r * D + pos * EPC]);
      if (q0 + r < n) {
        T* op = static_cast<T*>(a.out) +
                (static_cast<int64_t>(q_begin + q0 + r) * a.num_q_heads + head) * D +
                (pos ^ (r % OCH)) * EPC;
        *reinterpret_cast<u32x4*>(op) = v;
      }
    }
  } else if (q0 + qi < n) {
    const float inv = 1.f / l_tot;
    T* op = static_cast<T*>(a.out) +
            (static_cast<int64_t>(q_begin + q0 + qi) * a.num_q_heads + head) * D;
#pragma unroll
    for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        store4<DT>(op + 32 * dt + 8 * g4 + 4 * hh, oacc[dt][4 * g4] * inv,
                   oacc[dt][4 * g4 + 1] * inv, oacc[dt][4 * g4 + 2] * inv,
                   oacc[dt][4 * g4 + 3] * inv);
  }
}

template <typename DT, int D, int GW, int PB>
nv_status launch_prefill(const PrefillArgs& a, int num_seqs, int max_seqlen_q, int num_tiles,
                         hipStream_t s) {
  constexpr int BN = DT::kBytes == 2 ? 64 : 32;
  const int heads_y = a.num_kv_heads * (a.group / GW);
  dim3 grid;
  if (a.tile_schedule) {
    if (num_tiles <= 0) return NV_OK;
    grid = dim3(heads_y, num_tiles, 1);
  } else {
    const int tiles = (max_seqlen_q + 32 * PB - 1) / (32 * PB);
    if (tiles <= 0) return NV_OK;
    grid = dim3(tiles, heads_y, num_seqs);
  }
  if (a.bs_shift >= 0)
    paged_prefill_kernel<DT, D, GW, PB, BN, 1><<<grid, dim3(64 * GW * PB), 0, s>>>(a);
  else
    paged_prefill_kernel<DT, D, GW, PB, BN, 0><<<grid, dim3(64 * GW * PB), 0, s>>>(a);
  return nvp_host::launch_status();
}

// Eight waves per workgroup: the GQA group's heads times query-position blocks.
template <typename DT, int D>
nv_status dispatch_prefill(const PrefillArgs& a, int num_seqs, int max_seqlen_q, int num_tiles,
                           hipStream_t s) {
  switch (a.group) {
    case 1: return launch_prefill<DT, D, 1, 8>(a, num_seqs, max_seqlen_q, num_tiles, s);
    case 2: return launch_prefill<DT, D, 2, 4>(a, num_seqs, max_seqlen_q, num_tiles, s);
    case 4: return launch_prefill<DT, D, 4, 2>(a, num_seqs, max_seqlen_q, num_tiles, s);
    case 8: return launch_prefill<DT, D, 8, 1>(a, num_seqs, max_seqlen_q, num_tiles, s);
    default: return NV_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" int32_t nv_paged_prefill_tile_rows(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return 0;
  return 32 * (8 / g);  // eight waves: g heads x (8 / g) blocks of 32 query rows
}

extern "C" nv_status nv_paged_prefill(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                      int32_t max_seqlen_k, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, int32_t num_seqs,
                                      const int32_t* tile_schedule, int32_t num_tiles,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t num_blocks, int32_t block_size, float softmax_scale,
                                      int32_t causal, int32_t dtype, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 ||
      num_tiles < 0)
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
  if (num_seqs == 0 || max_seqlen_q == 0) return NV_OK;
  if (!out || !q || !k_cache || !v_cache || !cu_seqlens_q || !cu_seqlens_k || !block_tables)
    return NV_ERR_INVALID_ARG;
  if (max_seqlen_q > max_seqlen_k ||
      static_cast<int64_t>(max_seqlen_k) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return NV_ERR_INVALID_ARG;
  if (num_seqs > 65535 || static_cast<int64_t>(num_kv_heads) * g > 65535 || num_tiles > 65535)
    return NV_ERR_UNSUPPORTED;

  if (nvp_check::on()) {
    const nv_status st = nvp_check::prefill(
        cu_seqlens_q, cu_seqlens_k, block_tables, max_blocks_per_seq, num_seqs, block_size,
        num_blocks, max_seqlen_q, max_seqlen_k, tile_schedule, num_tiles,
        nv_paged_prefill_tile_rows(num_q_heads, num_kv_heads), stream);
    if (st != NV_OK) return st;
  }
  PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.block_tables = block_tables;
  a.tile_schedule = tile_schedule;
  a.max_blocks = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.group = g;
  a.causal = causal ? 1 : 0;
  a.bs_shift = nvp_host::is_pow2(block_size) ? __builtin_ctz(static_cast<unsigned>(block_size)) : -1;
  // The kernel takes a positive scale: a negative one flips the sign of q instead, and a
  // zero scale becomes 1e-30 (every score times it rounds to 0, so each weight is
  // exactly 2^0 = 1 as with scale 0, and masked keys stay at -inf).
  a.negate_q = softmax_scale < 0.f ? 1 : 0;
  const float mag = softmax_scale < 0.f ? -softmax_scale : softmax_scale;
  a.scale_log2 = mag > 0.f ? mag * 1.4426950408889634f : 1e-30f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == NV_BF16)
    return head_dim == 128 ? dispatch_prefill<BF16, 128>(a, num_seqs, max_seqlen_q, num_tiles, s)
                           : dispatch_prefill<BF16, 64>(a, num_seqs, max_seqlen_q, num_tiles, s);
  return head_dim == 128 ? dispatch_prefill<F32, 128>(a, num_seqs, max_seqlen_q, num_tiles, s)
                         : dispatch_prefill<F32, 64>(a, num_seqs, max_seqlen_q, num_tiles, s);
}
