// Host-side KV block manager: block tables, reference counts and prefix reuse.
//
// Walkthrough (xingyun3d.csdn.net nano-vllm article), section 五: a pool of fixed-size
// blocks with id, reference count, content hash and token ids; a hash index for prefix
// reuse; free and used sets.  allocate (prefill) walks a prompt block by block with a
// rolling hash, sharing hits and taking free blocks on misses; may_append (decode) opens
// a block at a block's first token and seals its hash when it is full; deallocate drops
// references and recycles blocks at zero.  Section 八: slot = block * block_size +
// offset.  The rules this file takes where the article is silent are listed in
// nvpaged_blocks.h.
//
// Layout: blocks live in one vector; the free pool is an intrusive doubly linked list
// threaded through them (first-in first-out, O(1) removal of any block, which a hit on a
// released block needs); sequences and the hash index are hash maps.
#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "nvpaged_blocks.h"

namespace {

// ---- XXH64, as specified in the xxHash documentation ------------------------------
constexpr uint64_t kPrime1 = 0x9E3779B185EBCA87ULL;
constexpr uint64_t kPrime2 = 0xC2B2AE3D27D4EB4FULL;
constexpr uint64_t kPrime3 = 0x165667B19E3779F9ULL;
constexpr uint64_t kPrime4 = 0x85EBCA77C2B2AE63ULL;
constexpr uint64_t kPrime5 = 0x27D4EB2F165667C5ULL;

inline uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

// Little-endian reads (the hosts this library runs on are little-endian).
inline uint64_t read64(const uint8_t* p) {
  uint64_t v;
  memcpy(&v, p, 8);
  return v;
}
inline uint32_t read32(const uint8_t* p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}

// One accumulator step on an 8-byte lane.
inline uint64_t lane_step(uint64_t acc, uint64_t lane) {
  return rotl64(acc + lane * kPrime2, 31) * kPrime1;
}

uint64_t xxh64(const uint8_t* p, size_t n, uint64_t seed) {
  const uint8_t* const end = p + n;
  uint64_t h;
  if (n >= 32) {  // four accumulators over 32-byte stripes, then converged
    uint64_t v[4] = {seed + kPrime1 + kPrime2, seed + kPrime2, seed, seed - kPrime1};
    for (; end - p >= 32; p += 32)
      for (int i = 0; i < 4; ++i) v[i] = lane_step(v[i], read64(p + 8 * i));
    h = rotl64(v[0], 1) + rotl64(v[1], 7) + rotl64(v[2], 12) + rotl64(v[3], 18);
    for (int i = 0; i < 4; ++i) h = (h ^ lane_step(0, v[i])) * kPrime1 + kPrime4;
  } else {
    h = seed + kPrime5;
  }
  h += static_cast<uint64_t>(n);
  for (; end - p >= 8; p += 8) h = rotl64(h ^ lane_step(0, read64(p)), 27) * kPrime1 + kPrime4;
  if (end - p >= 4) {
    h = rotl64(h ^ (static_cast<uint64_t>(read32(p)) * kPrime1), 23) * kPrime2 + kPrime3;
    p += 4;
  }
  for (; p < end; ++p) h = rotl64(h ^ (static_cast<uint64_t>(*p) * kPrime5), 11) * kPrime1;
  h ^= h >> 33;  // avalanche
  h *= kPrime2;
  h ^= h >> 29;
  h *= kPrime3;
  h ^= h >> 32;
  return h;
}

struct Block {
  int32_t ref = 0;
  bool hashed = false;
  uint64_t hash = 0;
  std::vector<int32_t> tokens;  // the tokens of a hashed (full) block
  int32_t prev = -1, next = -1;  // free-pool links
  bool in_pool = true;
};

struct Sequence {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  int32_t cached = 0;
  uint64_t stamp = 0;  // the batch call that last named this sequence (duplicate check)
};

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

}  // namespace

struct nv_block_manager {
  int32_t bs = 0;
  std::vector<Block> blocks;
  int32_t head = -1, tail = -1, nfree = 0;
  std::unordered_map<uint64_t, int32_t> index;
  std::unordered_map<int64_t, Sequence> seqs;
  std::vector<uint8_t> bytes;  // hash input scratch
  std::vector<Sequence*> batch_seqs;  // decode-step scratch
  uint64_t calls = 0;                 // batch-call counter for Sequence::stamp

  // ---- free pool ----------------------------------------------------------------
  void pool_push_back(int32_t id) {
    Block& b = blocks[id];
    b.prev = tail;
    b.next = -1;
    b.in_pool = true;
    if (tail >= 0) blocks[tail].next = id; else head = id;
    tail = id;
    ++nfree;
  }
  void pool_unlink(int32_t id) {
    Block& b = blocks[id];
    if (b.prev >= 0) blocks[b.prev].next = b.next; else head = b.next;
    if (b.next >= 0) blocks[b.next].prev = b.prev; else tail = b.prev;
    b.prev = b.next = -1;
    b.in_pool = false;
    --nfree;
  }
  // A block leaves the pool with one reference (a hit on a released block, or a miss).
  void take(int32_t id) {
    pool_unlink(id);
    blocks[id].ref = 1;
  }
  // A miss: the pool's front block, its previous content dropped.
  int32_t take_fresh() {
    const int32_t id = head;
    take(id);
    Block& b = blocks[id];
    if (b.hashed) {
      auto it = index.find(b.hash);
      if (it != index.end() && it->second == id) index.erase(it);
    }
    b.hashed = false;
    b.tokens.clear();
    return id;
  }

  // ---- hashing --------------------------------------------------------------------
  uint64_t block_hash(const int32_t* t, int32_t n, bool has_prev, uint64_t prev) {
    bytes.resize((has_prev ? 8 : 0) + 4 * static_cast<size_t>(n));
    uint8_t* p = bytes.data();
    if (has_prev) {
      for (int i = 0; i < 8; ++i) *p++ = static_cast<uint8_t>(prev >> (8 * i));
    }
    for (int32_t i = 0; i < n; ++i) {
      const uint32_t u = static_cast<uint32_t>(t[i]);
      for (int k = 0; k < 4; ++k) *p++ = static_cast<uint8_t>(u >> (8 * k));
    }
    return xxh64(bytes.data(), bytes.size(), 0);
  }
  void seal(int32_t id, const int32_t* t, uint64_t h) {
    Block& b = blocks[id];
    b.hashed = true;
    b.hash = h;
    b.tokens.assign(t, t + bs);
    index[h] = id;  // the latest block with this hash is the index entry
  }

  // ---- the article's operations (arguments already checked) -------------------------
  int32_t allocate(int64_t seq_id, const int32_t* t, int32_t n) {
    Sequence& s = seqs[seq_id];
    s.tokens.assign(t, t + n);
    const int32_t nblk = static_cast<int32_t>(blocks_for(n, bs));
    s.table.reserve(nblk);
    bool has_prev = false, missed = false;
    uint64_t prev = 0;
    for (int32_t i = 0; i < nblk; ++i) {
      const int32_t* bt = t + static_cast<int64_t>(i) * bs;
      const int32_t len = (i + 1 < nblk) ? bs : n - i * bs;
      const bool full = len == bs;
      const uint64_t h = full ? block_hash(bt, bs, has_prev, prev) : 0;
      int32_t hit = -1;
      if (full && i + 1 < nblk && !missed) {
        auto it = index.find(h);
        if (it != index.end() &&
            memcmp(blocks[it->second].tokens.data(), bt, sizeof(int32_t) * bs) == 0)
          hit = it->second;
      }
      if (hit >= 0) {
        s.cached += bs;
        if (blocks[hit].in_pool) take(hit); else ++blocks[hit].ref;
        s.table.push_back(hit);
      } else {
        missed = true;
        const int32_t id = take_fresh();
        if (full) seal(id, bt, h);
        s.table.push_back(id);
      }
      has_prev = full;
      prev = h;
    }
    return s.cached;
  }

  void append(Sequence& s, int32_t token) {
    s.tokens.push_back(token);
    const int64_t n = static_cast<int64_t>(s.tokens.size());
    if ((n - 1) % bs == 0) s.table.push_back(take_fresh());  // the token opens a block
    if (n % bs == 0) {                                         // the last block is full
      const size_t nb = s.table.size();
      const bool has_prev = nb > 1;
      const uint64_t prev = has_prev ? blocks[s.table[nb - 2]].hash : 0;
      const int32_t* t = s.tokens.data() + (n - bs);
      seal(s.table[nb - 1], t, block_hash(t, bs, has_prev, prev));
    }
  }

  void release(int64_t seq_id) {
    auto it = seqs.find(seq_id);
    const std::vector<int32_t>& table = it->second.table;
    for (size_t k = table.size(); k-- > 0;) {
      const int32_t id = table[k];
      if (--blocks[id].ref == 0) pool_push_back(id);
    }
    seqs.erase(it);
  }

  // New blocks that appending one token to s takes.
  int32_t append_need(const Sequence& s) const {
    return (static_cast<int64_t>(s.tokens.size()) % bs == 0) ? 1 : 0;
  }

  void write_row(const Sequence& s, int32_t* row, int32_t width) const {
    const int32_t nb = static_cast<int32_t>(s.table.size());
    for (int32_t i = 0; i < width; ++i) row[i] = i < nb ? s.table[i] : -1;
  }
};

namespace {

template <typename F>
nv_status guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {  // host memory exhausted: report, do not unwind into C
    return NV_ERR_INVALID_ARG;
  }
}

}  // namespace

extern "C" {

uint64_t nv_bm_xxh64(const void* data, int64_t n, uint64_t seed) {
  if (n <= 0 || data == nullptr) return xxh64(nullptr, 0, seed);
  return xxh64(static_cast<const uint8_t*>(data), static_cast<size_t>(n), seed);
}

nv_status nv_bm_create(int32_t num_blocks, int32_t block_size, nv_block_manager** out) {
  if (out == nullptr || num_blocks < 1 || block_size < 1) return NV_ERR_INVALID_ARG;
  *out = nullptr;
  return guarded([&] {
    nv_block_manager* bm = new nv_block_manager();
    bm->bs = block_size;
    bm->blocks.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->pool_push_back(i);
    *out = bm;
    return NV_OK;
  });
}

void nv_bm_destroy(nv_block_manager* bm) { delete bm; }

int32_t nv_bm_num_free_blocks(const nv_block_manager* bm) { return bm ? bm->nfree : 0; }

nv_status nv_bm_can_allocate(const nv_block_manager* bm, int32_t num_tokens, int32_t* ok) {
  if (bm == nullptr || ok == nullptr || num_tokens < 0) return NV_ERR_INVALID_ARG;
  *ok = bm->nfree >= blocks_for(num_tokens, bm->bs) ? 1 : 0;
  return NV_OK;
}

nv_status nv_bm_allocate(nv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                         int32_t num_tokens, int32_t* num_cached_tokens) {
  if (bm == nullptr || token_ids == nullptr || num_tokens < 1) return NV_ERR_INVALID_ARG;
  if (bm->seqs.count(seq_id)) return NV_ERR_INVALID_ARG;
  if (bm->nfree < blocks_for(num_tokens, bm->bs)) return NV_ERR_OUT_OF_BLOCKS;
  return guarded([&] {
    const int32_t c = bm->allocate(seq_id, token_ids, num_tokens);
    if (num_cached_tokens) *num_cached_tokens = c;
    return NV_OK;
  });
}

nv_status nv_bm_can_append(const nv_block_manager* bm, int64_t seq_id, int32_t* ok) {
  if (bm == nullptr || ok == nullptr) return NV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return NV_ERR_INVALID_ARG;
  *ok = bm->nfree >= bm->append_need(it->second) ? 1 : 0;
  return NV_OK;
}

nv_status nv_bm_append_token(nv_block_manager* bm, int64_t seq_id, int32_t token_id) {
  if (bm == nullptr) return NV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return NV_ERR_INVALID_ARG;
  if (bm->nfree < bm->append_need(it->second)) return NV_ERR_OUT_OF_BLOCKS;
  return guarded([&] {
    bm->append(it->second, token_id);
    return NV_OK;
  });
}

nv_status nv_bm_deallocate(nv_block_manager* bm, int64_t seq_id) {
  if (bm == nullptr || !bm->seqs.count(seq_id)) return NV_ERR_INVALID_ARG;
  bm->release(seq_id);
  return NV_OK;
}

nv_status nv_bm_get_sequence(const nv_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                             int32_t* num_cached_tokens, int32_t* table, int32_t capacity,
                             int32_t* num_blocks) {
  if (bm == nullptr) return NV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return NV_ERR_INVALID_ARG;
  const Sequence& s = it->second;
  const int32_t nb = static_cast<int32_t>(s.table.size());
  if (table != nullptr && capacity < nb) return NV_ERR_INVALID_ARG;
  if (num_tokens) *num_tokens = static_cast<int32_t>(s.tokens.size());
  if (num_cached_tokens) *num_cached_tokens = s.cached;
  if (num_blocks) *num_blocks = nb;
  if (table) memcpy(table, s.table.data(), sizeof(int32_t) * nb);
  return NV_OK;
}

nv_status nv_bm_get_block(const nv_block_manager* bm, int32_t block_id, int32_t* ref_count,
                          int32_t* has_hash, uint64_t* hash) {
  if (bm == nullptr || block_id < 0 || block_id >= static_cast<int32_t>(bm->blocks.size()))
    return NV_ERR_INVALID_ARG;
  const Block& b = bm->blocks[block_id];
  if (ref_count) *ref_count = b.ref;
  if (has_hash) *has_hash = b.hashed ? 1 : 0;
  if (hash) *hash = b.hashed ? b.hash : 0;
  return NV_OK;
}

nv_status nv_bm_get_free_blocks(const nv_block_manager* bm, int32_t* ids, int32_t capacity,
                                int32_t* count) {
  if (bm == nullptr || count == nullptr) return NV_ERR_INVALID_ARG;
  *count = bm->nfree;
  if (ids == nullptr) return NV_OK;
  if (capacity < bm->nfree) return NV_ERR_INVALID_ARG;
  int32_t k = 0;
  for (int32_t id = bm->head; id >= 0; id = bm->blocks[id].next) ids[k++] = id;
  return NV_OK;
}

nv_status nv_bm_decode_step(nv_block_manager* bm, const int64_t* seq_ids,
                            const int32_t* new_tokens, int32_t batch, int32_t* block_tables,
                            int32_t table_width, int32_t* context_lens,
                            int32_t* slot_mapping) {
  if (bm == nullptr || batch < 0 || table_width < 1) return NV_ERR_INVALID_ARG;
  if (batch == 0) return NV_OK;
  if (!seq_ids || !new_tokens || !block_tables || !context_lens || !slot_mapping)
    return NV_ERR_INVALID_ARG;
  return guarded([&] {
    std::vector<Sequence*>& seq = bm->batch_seqs;
    seq.resize(batch);
    const uint64_t stamp = ++bm->calls;
    int64_t need = 0;
    for (int32_t b = 0; b < batch; ++b) {
      auto it = bm->seqs.find(seq_ids[b]);
      if (it == bm->seqs.end() || it->second.stamp == stamp) return NV_ERR_INVALID_ARG;
      it->second.stamp = stamp;
      seq[b] = &it->second;
      if (blocks_for(static_cast<int64_t>(seq[b]->tokens.size()) + 1, bm->bs) > table_width)
        return NV_ERR_INVALID_ARG;
      need += bm->append_need(*seq[b]);
    }
    if (need > bm->nfree) return NV_ERR_OUT_OF_BLOCKS;
    const int32_t bs = bm->bs;
    for (int32_t b = 0; b < batch; ++b) {
      Sequence& s = *seq[b];
      bm->append(s, new_tokens[b]);
      const int32_t len = static_cast<int32_t>(s.tokens.size());
      const int32_t pos = len - 1;
      bm->write_row(s, block_tables + static_cast<int64_t>(b) * table_width, table_width);
      context_lens[b] = len;
      slot_mapping[b] = s.table[pos / bs] * bs + pos % bs;
    }
    return NV_OK;
  });
}

nv_status nv_bm_prefill_step(nv_block_manager* bm, const int64_t* seq_ids,
                             const int32_t* cu_tokens, const int32_t* token_ids,
                             int32_t num_seqs, int32_t* block_tables, int32_t table_width,
                             int32_t* num_cached) {
  if (bm == nullptr || num_seqs < 0 || table_width < 1) return NV_ERR_INVALID_ARG;
  if (num_seqs == 0) return NV_OK;
  if (!seq_ids || !cu_tokens || !token_ids || !block_tables || !num_cached)
    return NV_ERR_INVALID_ARG;
  return guarded([&] {
    std::unordered_set<int64_t> seen;
    seen.reserve(num_seqs * 2);
    int64_t need = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int64_t n = static_cast<int64_t>(cu_tokens[s + 1]) - cu_tokens[s];
      if (cu_tokens[s] < 0 || n < 1 || bm->seqs.count(seq_ids[s]) ||
          !seen.insert(seq_ids[s]).second || blocks_for(n, bm->bs) > table_width)
        return NV_ERR_INVALID_ARG;
      need += blocks_for(n, bm->bs);
    }
    if (need > bm->nfree) return NV_ERR_OUT_OF_BLOCKS;
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t n = cu_tokens[s + 1] - cu_tokens[s];
      num_cached[s] = bm->allocate(seq_ids[s], token_ids + cu_tokens[s], n);
      bm->write_row(bm->seqs[seq_ids[s]], block_tables + static_cast<int64_t>(s) * table_width,
                    table_width);
    }
    return NV_OK;
  });
}

}  // extern "C"
