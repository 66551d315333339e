// Host-side descriptor builder and block cache (see include/minipic_desc.h).
// The hashing rule and the segment semantics follow "MiniPIC: Flexible
// Position-Independent Caching in <100LOC", §3.1.1 (the three primitives and
// the block hash recurrence) and §3.3.1 / §3.3.2 (how Block-Attention and EPIC
// place the markers).
#include <cstdint>
#include <cstdio>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/minipic_desc.h"

namespace minipic_host {
// set by the attention library's error helper (same thread-local slot)
int set_error(int code, const std::string& msg);
}

namespace {

constexpr int kBlock = 16;

// SplitMix64 output function (Steele, Lea and Flood, 2014).
inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// H(h, x): fold the tokens of x into h one at a time.
inline uint64_t fold(uint64_t h, const int32_t* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h = mix((h ^ (uint64_t)(uint32_t)x[i]) + 0x9E3779B97F4A7C15ull);
  return h;
}

inline bool is(int32_t tok, int32_t marker) { return marker >= 0 && tok == marker; }

}  // namespace

struct minipic_block_cache {
  std::unordered_map<uint64_t, int32_t> map;
  std::vector<int32_t> free_list;   // physical blocks not yet handed out (popped from the back)
};

extern "C" {

int minipic_describe_blocks(const int32_t* tokens, int64_t n, const minipic_markers* m, int32_t block_size,
                            uint64_t* hashes, int32_t* span_id, uint8_t* flags, int64_t max_blocks,
                            int64_t* num_blocks) {
  using minipic_host::set_error;
  if (!m || !num_blocks || (n > 0 && (!tokens || !hashes || !span_id || !flags)))
    return set_error(MINIPIC_ERR_INVALID_ARG, "NULL argument");
  if (n < 0) return set_error(MINIPIC_ERR_INVALID_ARG, "n < 0");
  if (block_size != kBlock) return set_error(MINIPIC_ERR_UNSUPPORTED, "block_size must be 16");
  const int64_t nb = (n + kBlock - 1) / kBlock;
  if (max_blocks < nb) return set_error(MINIPIC_ERR_INVALID_ARG, "max_blocks is smaller than ceil(n / 16)");
  // contract: a marker only as the first token of a block
  for (int64_t t = 0; t < n; ++t) {
    const int32_t x = tokens[t];
    if ((is(x, m->ssep) || is(x, m->pdep) || is(x, m->global_)) && t % kBlock != 0) {
      char buf[160];
      snprintf(buf, sizeof buf, "marker token %d at position %lld is not the first token of a 16-token block "
               "(pad the previous segment)", (int)x, (long long)t);
      return set_error(MINIPIC_ERR_CONTRACT, buf);
    }
  }
  uint64_t h_prev = m->seed;   // h_{i-1}
  uint64_t g = m->seed;        // H(h_0, x_<=i): every token so far
  // Hash of the last GLOBAL block so far (h_0 before the first). Tokens of a
  // span attend to every earlier GLOBAL block, so from the second layer on
  // their K/V depend on that prefix: a span (or a later GLOBAL segment)
  // chains from it instead of h_0, and the same document after a different
  // shared prefix does not hit.
  uint64_t anchor = m->seed;
  int32_t span = 0;
  uint8_t seg_flags = 0;
  for (int64_t i = 0; i < nb; ++i) {
    const int32_t* x = tokens + i * kBlock;
    const int64_t len = (i + 1) * kBlock <= n ? kBlock : n - i * kBlock;
    g = fold(g, x, len);
    uint64_t h;
    if (is(x[0], m->ssep) || is(x[0], m->global_)) {
      h = fold(anchor, x, len);
    } else if (is(x[0], m->pdep)) {
      h = g;
    } else {
      h = fold(h_prev, x, len);
    }
    if (i > 0 && (is(x[0], m->ssep) || is(x[0], m->pdep) || is(x[0], m->global_))) ++span;
    if (is(x[0], m->ssep)) seg_flags = 0;
    if (is(x[0], m->pdep)) seg_flags = MINIPIC_BLK_PDEP;
    if (is(x[0], m->global_)) seg_flags = MINIPIC_BLK_GLOBAL;
    hashes[i] = h;
    span_id[i] = span;
    flags[i] = seg_flags;
    h_prev = h;
    if (seg_flags & MINIPIC_BLK_GLOBAL) anchor = h;
  }
  *num_blocks = nb;
  return MINIPIC_OK;
}

minipic_block_cache* minipic_block_cache_create(int64_t num_blocks) {
  if (num_blocks <= 0 || num_blocks > INT32_MAX) return nullptr;
  try {
    auto* c = new minipic_block_cache;
    c->free_list.resize((size_t)num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) c->free_list[(size_t)i] = (int32_t)(num_blocks - 1 - i);
    return c;
  } catch (...) {
    return nullptr;
  }
}

void minipic_block_cache_destroy(minipic_block_cache* cache) { delete cache; }

int minipic_block_cache_assign(minipic_block_cache* c, const uint64_t* hashes, int64_t nb, int32_t* block_table,
                               uint8_t* hit, int64_t* num_hits) {
  using minipic_host::set_error;
  if (!c || !num_hits || (nb > 0 && (!hashes || !block_table || !hit)))
    return set_error(MINIPIC_ERR_INVALID_ARG, "NULL argument");
  if (nb < 0) return set_error(MINIPIC_ERR_INVALID_ARG, "nb < 0");
  // count the new hashes first so that a full cache records nothing
  std::unordered_set<uint64_t> fresh;
  for (int64_t i = 0; i < nb; ++i)
    if (!c->map.count(hashes[i])) fresh.insert(hashes[i]);
  if ((int64_t)fresh.size() > (int64_t)c->free_list.size())
    return set_error(MINIPIC_ERR_CACHE_FULL, "block cache has too few free blocks");
  int64_t hits = 0;
  for (int64_t i = 0; i < nb; ++i) {
    auto it = c->map.find(hashes[i]);
    if (it != c->map.end()) {   // cached before, or taken by an earlier block of this request
      block_table[i] = it->second;
      hit[i] = 1;
      ++hits;
    } else {
      const int32_t b = c->free_list.back();
      c->free_list.pop_back();
      c->map.emplace(hashes[i], b);
      block_table[i] = b;
      hit[i] = 0;
    }
  }
  *num_hits = hits;
  return MINIPIC_OK;
}

int minipic_slot_mapping(const int32_t* block_table, const uint8_t* hit, int64_t n, int32_t block_size,
                         int64_t* slots, int32_t* ctx_index, int64_t* count) {
  using minipic_host::set_error;
  if (!count || (n > 0 && (!block_table || !hit || !slots))) return set_error(MINIPIC_ERR_INVALID_ARG, "NULL argument");
  if (n < 0) return set_error(MINIPIC_ERR_INVALID_ARG, "n < 0");
  if (block_size != kBlock) return set_error(MINIPIC_ERR_UNSUPPORTED, "block_size must be 16");
  int64_t k = 0;
  for (int64_t t = 0; t < n; ++t) {
    const int64_t i = t / kBlock;
    if (hit[i]) continue;
    slots[k] = (int64_t)block_table[i] * kBlock + t % kBlock;
    if (ctx_index) ctx_index[k] = (int32_t)t;
    ++k;
  }
  *count = k;
  return MINIPIC_OK;
}

}  // extern "C"
