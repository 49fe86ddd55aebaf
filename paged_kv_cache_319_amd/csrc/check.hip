// Check mode: validation of the device-data preconditions of the entry points.
//
// The kernels trust the values inside device arrays (slots, block ids, lengths,
// cu_seqlens, schedules): checking them on every call would cost a pass over
// metadata and a host synchronisation.  With check mode on (environment variable
// NV_CHECK=1 at the first call, or nv_set_check_mode(1)), each GPU entry point
// first runs the kernels below on its stream, waits for them, and returns
// NV_ERR_INVALID_ARG without launching its own work if any precondition fails;
// nv_check_message() then describes one failure: the lowest-numbered kind of
// violation found, at its lowest element index.  Every check reads only the elements the arguments say
// exist, so a violation found here never becomes an out-of-bounds access.
//
// The preconditions follow the walkthrough (xingyun3d.csdn.net nano-vllm
// article), sections 七 and 八: a slot is block * block_size + offset of a
// physical row, a block table lists a sequence's physical blocks, cu_seqlens are
// prefix sums of the query and key counts.
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"

namespace {

// Smallest (kind, index) key reported by any thread of the current check:
// kind in the top byte, element index below it.  ~0 = no violation.
__device__ unsigned long long g_first_violation;
// Number of tiles the sequences hold, summed by the prefill check when a tile
// schedule is given (it must list every one of them).
__device__ unsigned long long g_tile_total;

enum Kind : unsigned {
  kSlotRange = 1,
  kSlotDuplicate,
  kLength,
  kBlockId,
  kSchedule,
  kCuSeqlensQ,
  kCuSeqlensK,
  kKeysFewerThanQueries,
  kSeqlenBound,
  kTileSchedule,
  kNewSlot,
  kTemperature,
};

const char* kind_name(unsigned k) {
  switch (k) {
    case kSlotRange: return "slot outside [0, num_blocks * block_size) and not -1";
    case kSlotDuplicate: return "slot used by two rows";
    case kLength: return "context length outside [1, min(max_context_len, table width * block_size)]";
    case kBlockId: return "block-table entry of a used block outside [0, num_blocks)";
    case kSchedule: return "schedule entry outside [0, batch) or repeated";
    case kCuSeqlensQ: return "cu_seqlens_q does not start at 0 or decreases";
    case kCuSeqlensK: return "cu_seqlens_k does not start at 0 or decreases";
    case kKeysFewerThanQueries: return "sequence with fewer keys than queries";
    case kSeqlenBound: return "sequence longer than max_seqlen_q / max_seqlen_k";
    case kTileSchedule: return "tile schedule entry names no tile of a sequence, repeats one, or misses one";
    case kNewSlot: return "slot_mapping[b] is neither -1 nor the slot of position context_lens[b] - 1";
    case kTemperature: return "temperature negative, infinite or NaN";
    default: return "unknown";
  }
}

__device__ __forceinline__ void report(unsigned kind, long long index) {
  const unsigned long long key =
      (static_cast<unsigned long long>(kind) << 56) | static_cast<unsigned long long>(index);
  atomicMin(&g_first_violation, key);
}

constexpr int kThreads = 256;
// Pairwise duplicate checks are quadratic; longer arrays get the range checks only.
constexpr int64_t kMaxPairwise = 1 << 16;

__global__ __launch_bounds__(kThreads) void check_slots_kernel(const int32_t* slots, int32_t n,
                                                               int64_t limit, bool pairwise) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  const int32_t s = slots[i];
  if (s == -1) return;
  if (s < 0 || s >= limit) {
    report(kSlotRange, i);
    return;
  }
  if (!pairwise) return;
  for (int64_t j = i + 1; j < n; ++j)
    if (slots[j] == s) {
      report(kSlotDuplicate, j);
      return;
    }
}

// One thread per sequence: its length, the table entries of its used blocks, its
// schedule entry and, for the fused store, its new-token slot.
__global__ __launch_bounds__(kThreads) void check_decode_kernel(
    const int32_t* tables, int32_t width, const int32_t* lens, const int32_t* schedule,
    const int32_t* new_slots, int32_t batch, int32_t block_size, int32_t num_blocks,
    int32_t max_len, bool pairwise) {
  const int32_t b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= batch) return;
  if (schedule) {
    const int32_t v = schedule[b];
    if (v < 0 || v >= batch) {
      report(kSchedule, b);
    } else if (pairwise) {
      for (int32_t j = b + 1; j < batch; ++j)
        if (schedule[j] == v) {
          report(kSchedule, j);
          break;
        }
    }
  }
  const int32_t L = lens[b];
  if (L < 1 || L > max_len || static_cast<int64_t>(L) > static_cast<int64_t>(width) * block_size) {
    report(kLength, b);
    return;
  }
  const int32_t* row = tables + static_cast<int64_t>(b) * width;
  const int32_t used = (L + block_size - 1) / block_size;
  for (int32_t e = 0; e < used; ++e) {
    const int32_t blk = row[e];
    if (blk < 0 || blk >= num_blocks) {
      report(kBlockId, b);
      return;
    }
  }
  if (new_slots) {
    const int32_t s = new_slots[b];
    const int32_t pos = L - 1;
    const int64_t want = static_cast<int64_t>(row[pos / block_size]) * block_size + pos % block_size;
    if (s != -1 && s != want) report(kNewSlot, b);
  }
}

// One thread per sequence: cu_seqlens shape, bounds and the used table entries.
__global__ __launch_bounds__(kThreads) void check_prefill_kernel(
    const int32_t* cu_q, const int32_t* cu_k, const int32_t* tables, int32_t width,
    int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t max_q, int32_t max_k,
    int32_t tile_rows) {
  const int32_t s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= num_seqs) return;
  if (s == 0 && cu_q[0] != 0) report(kCuSeqlensQ, 0);
  if (s == 0 && cu_k[0] != 0) report(kCuSeqlensK, 0);
  const int32_t nq = cu_q[s + 1] - cu_q[s];
  const int32_t nk = cu_k[s + 1] - cu_k[s];
  if (tile_rows > 0 && nq > 0)
    atomicAdd(&g_tile_total, static_cast<unsigned long long>((nq + tile_rows - 1) / tile_rows));
  if (nq < 0) {
    report(kCuSeqlensQ, s + 1);
    return;
  }
  if (nk < 0) {
    report(kCuSeqlensK, s + 1);
    return;
  }
  if (nk < nq) {
    report(kKeysFewerThanQueries, s);
    return;
  }
  if (nq > max_q || nk > max_k || static_cast<int64_t>(nk) > static_cast<int64_t>(width) * block_size) {
    report(kSeqlenBound, s);
    return;
  }
  const int32_t* row = tables + static_cast<int64_t>(s) * width;
  const int32_t used = (nk + block_size - 1) / block_size;
  for (int32_t e = 0; e < used; ++e) {
    const int32_t blk = row[e];
    if (blk < 0 || blk >= num_blocks) {
      report(kBlockId, s);
      return;
    }
  }
}

// One thread per tile-schedule pair: a (sequence, tile) that exists, listed once.
__global__ __launch_bounds__(kThreads) void check_tiles_kernel(const int32_t* tiles,
                                                               int32_t num_tiles,
                                                               const int32_t* cu_q,
                                                               int32_t num_seqs, int32_t rows,
                                                               bool pairwise) {
  const int32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= num_tiles) return;
  const int32_t s = tiles[2 * i], t = tiles[2 * i + 1];
  if (s < 0 || s >= num_seqs || t < 0) {
    report(kTileSchedule, i);
    return;
  }
  const int32_t nq = cu_q[s + 1] - cu_q[s];
  if (static_cast<int64_t>(t) * rows >= nq) {
    report(kTileSchedule, i);
    return;
  }
  if (!pairwise) return;
  for (int32_t j = i + 1; j < num_tiles; ++j)
    if (tiles[2 * j] == s && tiles[2 * j + 1] == t) {
      report(kTileSchedule, j);
      return;
    }
}

__global__ __launch_bounds__(kThreads) void check_temperatures_kernel(const float* t,
                                                                      int32_t batch) {
  const int32_t b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= batch) return;
  const float v = t[b];
  if (!(v >= 0.0f) || v == INFINITY) report(kTemperature, b);
}

__global__ void check_tile_count_kernel(int32_t num_tiles) {
  if (threadIdx.x == 0 && g_tile_total != static_cast<unsigned long long>(num_tiles))
    report(kTileSchedule, num_tiles);
}

std::mutex g_check_mutex;  // one check at a time per process: they share the device flag
int g_mode = -1;           // -1: not read from the environment yet
thread_local char g_message[256] = "no violation";

bool check_enabled() {
  std::lock_guard<std::mutex> lock(g_check_mutex);
  if (g_mode < 0) {
    const char* e = getenv("NV_CHECK");
    g_mode = (e && e[0] && strcmp(e, "0") != 0) ? 1 : 0;
  }
  return g_mode == 1;
}

unsigned grid_for(int64_t n) { return static_cast<unsigned>((n + kThreads - 1) / kThreads); }

// Resets the process-wide check state on the stream: no violation found yet and, for a
// prefill check with a tile schedule, no tiles counted yet.
__global__ void reset_check_state_kernel(bool tiles) {
  if (threadIdx.x == 0) {
    g_first_violation = ~0ull;
    if (tiles) g_tile_total = 0;
  }
}

// Under the process-wide lock (the device flags are shared by every check of the
// process): resets the flags, runs `launch` on the stream, waits, and reads the first
// violation back.
template <typename F>
nv_status run_check(const char* what, hipStream_t s, bool reset_tiles, F launch) {
  std::lock_guard<std::mutex> lock(g_check_mutex);
  const unsigned long long none = ~0ull;
  reset_check_state_kernel<<<1, 64, 0, s>>>(reset_tiles);
  launch();
  if (hipGetLastError() != hipSuccess) return NV_ERR_HIP;
  unsigned long long first = none;
  if (hipMemcpyFromSymbolAsync(&first, HIP_SYMBOL(g_first_violation), sizeof(first), 0,
                               hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return NV_ERR_HIP;
  if (first == none) {
    snprintf(g_message, sizeof(g_message), "no violation");
    return NV_OK;
  }
  const unsigned kind = static_cast<unsigned>(first >> 56);
  const long long index = static_cast<long long>(first & ((1ull << 56) - 1));
  snprintf(g_message, sizeof(g_message), "%s: %s (element %lld)", what, kind_name(kind), index);
  return NV_ERR_INVALID_ARG;
}

}  // namespace

namespace nvp_check {

bool on() { return check_enabled(); }

nv_status store(const int32_t* slots, int32_t n, int32_t num_blocks, int32_t block_size,
                void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t limit = static_cast<int64_t>(num_blocks) * block_size;
  return run_check("nv_store_kvcache", s, false, [&] {
    check_slots_kernel<<<grid_for(n), kThreads, 0, s>>>(slots, n, limit, n <= kMaxPairwise);
  });
}

nv_status decode(const int32_t* tables, int32_t width, const int32_t* lens,
                 const int32_t* schedule, const int32_t* new_slots, int32_t batch,
                 int32_t block_size, int32_t num_blocks, int32_t max_len, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t limit = static_cast<int64_t>(num_blocks) * block_size;
  return run_check(new_slots ? "nv_paged_decode_store" : "nv_paged_decode", s, false, [&] {
    check_decode_kernel<<<grid_for(batch), kThreads, 0, s>>>(tables, width, lens, schedule,
                                                             new_slots, batch, block_size,
                                                             num_blocks, max_len,
                                                             batch <= kMaxPairwise);
    if (new_slots)
      check_slots_kernel<<<grid_for(batch), kThreads, 0, s>>>(new_slots, batch, limit,
                                                              batch <= kMaxPairwise);
  });
}

nv_status prefill(const int32_t* cu_q, const int32_t* cu_k, const int32_t* tables, int32_t width,
                  int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t max_q,
                  int32_t max_k, const int32_t* tiles, int32_t num_tiles, int32_t tile_rows,
                  void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool with_tiles = tiles && num_tiles > 0;
  return run_check("nv_paged_prefill", s, with_tiles, [&] {
    check_prefill_kernel<<<grid_for(num_seqs), kThreads, 0, s>>>(
        cu_q, cu_k, tables, width, num_seqs, block_size, num_blocks, max_q, max_k,
        with_tiles ? tile_rows : 0);
    if (with_tiles) {
      check_tiles_kernel<<<grid_for(num_tiles), kThreads, 0, s>>>(
          tiles, num_tiles, cu_q, num_seqs, tile_rows, num_tiles <= kMaxPairwise);
      check_tile_count_kernel<<<1, 64, 0, s>>>(num_tiles);
    }
  });
}

nv_status sample(const float* temperatures, int32_t batch, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return run_check("nv_sample", s, false, [&] {
    check_temperatures_kernel<<<grid_for(batch), kThreads, 0, s>>>(temperatures, batch);
  });
}

}  // namespace nvp_check

extern "C" int32_t nv_set_check_mode(int32_t on) {
  const bool prev = check_enabled();  // reads NV_CHECK on first use
  std::lock_guard<std::mutex> lock(g_check_mutex);
  g_mode = on ? 1 : 0;
  return prev ? 1 : 0;
}

extern "C" const char* nv_check_message(void) { return g_message; }
