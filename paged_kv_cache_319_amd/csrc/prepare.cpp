// Host-side step metadata: slot_mapping and cu_seqlens.
//
// Walkthrough (xingyun3d.csdn.net nano-vllm article), section 七: before each
// forward pass the runner builds, for prefill, the prefix sums cu_seqlens_q/k,
// max_seqlen_q/k and the physical slot of every newly written token; for
// decode, each sequence's current length and the slot of its last token.
// Section 八 defines the slot as the one-dimensional index of the physical row;
// the gsyq.cn paging article (section 4.1) places token t in logical block
// t / B at offset t % B.  With the cache viewed as [num_blocks * B, ...] rows,
// slot = block_tables[s][t / B] * B + t % B.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "nvpaged.h"

namespace {

// Slot of position t of the sequence whose table row is `row`; -1 on a bad entry.
int64_t slot_for(const int32_t* row, int32_t width, int32_t t, int32_t block_size,
                 int32_t num_blocks) {
  const int32_t logical = t / block_size;
  if (t < 0 || logical >= width) return -1;
  const int32_t blk = row[logical];
  if (blk < 0 || blk >= num_blocks) return -1;
  return static_cast<int64_t>(blk) * block_size + t % block_size;
}

}  // namespace

extern "C" const char* nv_status_string(nv_status status) {
  switch (status) {
    case NV_OK: return "ok";
    case NV_ERR_INVALID_ARG: return "invalid argument";
    case NV_ERR_UNSUPPORTED: return "unsupported configuration";
    case NV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case NV_ERR_HIP: return "HIP runtime error";
    case NV_ERR_OUT_OF_BLOCKS: return "not enough free KV blocks";
  }
  return "unknown status";
}

extern "C" nv_status nv_prepare_decode(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t batch,
                                       int32_t block_size, int32_t num_blocks,
                                       int32_t* slot_mapping, int32_t* schedule,
                                       int32_t* max_context_len) {
  if (batch < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0 ||
      !max_context_len)
    return NV_ERR_INVALID_ARG;
  if (batch > 0 && (!block_tables || !context_lens || !slot_mapping)) return NV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return NV_ERR_UNSUPPORTED;
  int32_t mx = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t L = context_lens[b];
    if (L < 1) return NV_ERR_INVALID_ARG;
    const int64_t slot = slot_for(block_tables + static_cast<int64_t>(b) * max_blocks_per_seq,
                                  max_blocks_per_seq, L - 1, block_size, num_blocks);
    if (slot < 0) return NV_ERR_INVALID_ARG;
    slot_mapping[b] = static_cast<int32_t>(slot);
    if (L > mx) mx = L;
  }
  *max_context_len = mx;
  if (schedule) {
    // Sequences whose leading blocks other sequences of the batch hold too (a shared,
    // ref-counted prefix at the same logical positions) come first, those with more
    // shared leading blocks first, so that the sharers' reads of the same rows fall close
    // together in time and hit the caches; within that, the longest first, so that long
    // work items start before the short ones fill the tail.  Ties keep index order.
    auto nblk = [&](int32_t b) {
      const int32_t n = (context_lens[b] + block_size - 1) / block_size;
      return n < max_blocks_per_seq ? n : max_blocks_per_seq;
    };
    auto row = [&](int32_t b) { return block_tables + static_cast<int64_t>(b) * max_blocks_per_seq; };
    // Common leading entries of two rows (entries outside [0, num_blocks) never match).
    auto common = [&](int32_t x, int32_t y) {
      const int32_t n = std::min(nblk(x), nblk(y));
      int32_t i = 0;
      while (i < n && row(x)[i] == row(y)[i] && row(x)[i] >= 0 && row(x)[i] < num_blocks) ++i;
      return i;
    };
    // In lexicographic order of the rows, a sequence's longest common prefix with any
    // other sequence is with one of its neighbours.
    std::vector<int32_t> order(batch), lead(batch, 0);
    for (int32_t b = 0; b < batch; ++b) order[b] = b;
    std::sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
      const int32_t n = std::min(nblk(x), nblk(y));
      for (int32_t i = 0; i < n; ++i)
        if (row(x)[i] != row(y)[i]) return row(x)[i] < row(y)[i];
      return nblk(x) != nblk(y) ? nblk(x) < nblk(y) : x < y;
    });
    for (int32_t k = 0; k + 1 < batch; ++k) {
      const int32_t c = common(order[k], order[k + 1]);
      lead[order[k]] = std::max(lead[order[k]], c);
      lead[order[k + 1]] = std::max(lead[order[k + 1]], c);
    }
    for (int32_t b = 0; b < batch; ++b) schedule[b] = b;
    std::stable_sort(schedule, schedule + batch, [&](int32_t x, int32_t y) {
      if (lead[x] != lead[y]) return lead[x] > lead[y];
      return context_lens[x] > context_lens[y];
    });
  }
  return NV_OK;
}

extern "C" nv_status nv_prepare_prefill(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* num_cached, const int32_t* num_new,
                                        int32_t num_seqs, int32_t block_size, int32_t num_blocks,
                                        int32_t pad_to, int32_t* cu_seqlens_q,
                                        int32_t* cu_seqlens_k, int32_t* max_seqlen_q,
                                        int32_t* max_seqlen_k, int32_t* slot_mapping,
                                        int32_t slot_capacity, int32_t* num_slots,
                                        int32_t tile_rows, int32_t* tile_schedule,
                                        int32_t tile_capacity, int32_t* num_tiles) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0 ||
      pad_to < 1 || slot_capacity < 0)
    return NV_ERR_INVALID_ARG;
  if (!cu_seqlens_q || !cu_seqlens_k || !max_seqlen_q || !max_seqlen_k || !num_slots)
    return NV_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!block_tables || !num_cached || !num_new)) return NV_ERR_INVALID_ARG;
  if (slot_capacity > 0 && !slot_mapping) return NV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return NV_ERR_UNSUPPORTED;
  int64_t cq = 0, ck = 0, n = 0;
  int32_t mq = 0, mk = 0;
  cu_seqlens_q[0] = 0;
  cu_seqlens_k[0] = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t p = num_cached[s], nn = num_new[s];
    if (p < 0 || nn < 0) return NV_ERR_INVALID_ARG;
    const int32_t* row = block_tables + static_cast<int64_t>(s) * max_blocks_per_seq;
    for (int32_t t = p; t < p + nn; ++t) {
      const int64_t slot = slot_for(row, max_blocks_per_seq, t, block_size, num_blocks);
      if (slot < 0) return NV_ERR_INVALID_ARG;
      if (n >= slot_capacity) return NV_ERR_INVALID_ARG;
      slot_mapping[n++] = static_cast<int32_t>(slot);
    }
    cq += nn;
    ck += static_cast<int64_t>(p) + nn;
    if (cq > INT32_MAX || ck > INT32_MAX) return NV_ERR_INVALID_ARG;
    cu_seqlens_q[s + 1] = static_cast<int32_t>(cq);
    cu_seqlens_k[s + 1] = static_cast<int32_t>(ck);
    if (nn > mq) mq = nn;
    if (p + nn > mk) mk = p + nn;
  }
  const int64_t padded = (n + pad_to - 1) / pad_to * pad_to;
  if (padded > slot_capacity) return NV_ERR_INVALID_ARG;
  for (int64_t i = n; i < padded; ++i) slot_mapping[i] = -1;
  *max_seqlen_q = mq;
  *max_seqlen_k = mk;
  *num_slots = static_cast<int32_t>(padded);
  if (tile_schedule) {
    // Attention work tiles (tile_rows query rows of one sequence), heaviest first: a
    // tile's causal key count is num_cached + the end of its row range.
    if (tile_rows <= 0 || !num_tiles) return NV_ERR_INVALID_ARG;
    struct Tile { int64_t keys; int32_t seq, tile; };
    std::vector<Tile> tiles;
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t nn = num_new[s];
      for (int32_t t = 0; static_cast<int64_t>(t) * tile_rows < nn; ++t) {
        const int64_t end = std::min<int64_t>(static_cast<int64_t>(t + 1) * tile_rows, nn);
        tiles.push_back(Tile{num_cached[s] + end, s, t});
      }
    }
    if (static_cast<int64_t>(tiles.size()) > tile_capacity) return NV_ERR_INVALID_ARG;
    std::stable_sort(tiles.begin(), tiles.end(),
                     [](const Tile& x, const Tile& y) { return x.keys > y.keys; });
    for (size_t i = 0; i < tiles.size(); ++i) {
      tile_schedule[2 * i] = tiles[i].seq;
      tile_schedule[2 * i + 1] = tiles[i].tile;
    }
    *num_tiles = static_cast<int32_t>(tiles.size());
  } else if (num_tiles) {
    *num_tiles = 0;
  }
  return NV_OK;
}
