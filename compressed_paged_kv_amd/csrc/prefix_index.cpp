// Prefix index (host C++): full blocks of prompts, found again by content.
//
// Prefix caching lets requests that start with the same tokens share the
// physical blocks holding them (upskillscore.com guide "Paged KV cache and
// continuous batching", "How it works": shared blocks with reference
// counts); the Zipage summaries keep it working next to compression (ko
// page "기술 요약" section 2.C, nl page "Technische samenvatting",
// Methodologie item 3).  An entry is one full block of b tokens, identified
// by its tokens and by the entry of the block before it, so a block matches
// only after the same whole prefix.  Lookups go through a 64-bit hash of
// (parent entry, tokens) and then compare the tokens themselves, so a hash
// collision never produces a false match.  The index holds one reference on
// every block it lists (the block survives the requests that filled it);
// least-recently-used entries without children are dropped on demand.
#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "block_pool.h"
#include "zp_internal.h"

namespace {

struct Entry {
  int32_t parent = -1;  // entry of the previous block, -1 for the first block
  int32_t block = -1;
  int32_t children = 0;
  int64_t last_used = 0;
  bool live = false;
  std::vector<int32_t> tokens;
};

uint64_t mix(uint64_t h, uint64_t x) {
  // splitmix64 finaliser over the running state
  h ^= x + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
  h ^= h >> 30;
  h *= 0xBF58476D1CE4E5B9ull;
  h ^= h >> 27;
  h *= 0x94D049BB133111EBull;
  h ^= h >> 31;
  return h;
}

uint64_t key_of(int32_t parent, const int32_t* tokens, int32_t b) {
  uint64_t h = mix(0x12345678u, (uint64_t)(uint32_t)parent);
  for (int32_t i = 0; i < b; i++) h = mix(h, (uint64_t)(uint32_t)tokens[i]);
  return h;
}

}  // namespace

struct zp_prefix_index {
  zp_block_pool* pool = nullptr;
  int32_t b = 0;
  int64_t clock = 0;
  std::vector<Entry> entries;
  std::vector<int32_t> free_entries;
  std::unordered_multimap<uint64_t, int32_t> by_key;
  int32_t live = 0;

  int32_t find(int32_t parent, const int32_t* tokens) const {
    auto range = by_key.equal_range(key_of(parent, tokens, b));
    for (auto it = range.first; it != range.second; ++it) {
      const Entry& e = entries[(size_t)it->second];
      if (e.live && e.parent == parent && std::memcmp(e.tokens.data(), tokens, (size_t)b * 4) == 0)
        return it->second;
    }
    return -1;
  }
};

extern "C" {

zp_status zp_prefix_index_create(zp_block_pool* pool, int32_t block_size, zp_prefix_index** out) {
  zp::clear_error();
  if (!pool || !out) { zp::set_error("pool and out must not be NULL"); return ZP_ERR_INVALID; }
  if (block_size < 1) { zp::set_error("block_size must be >= 1"); return ZP_ERR_INVALID; }
  zp_prefix_index* x = new zp_prefix_index();
  x->pool = pool;
  x->b = block_size;
  *out = x;
  return ZP_OK;
}

void zp_prefix_index_destroy(zp_prefix_index* x) {
  if (!x) return;
  // give back the index's references; blocks reaching 0 become free
  for (const Entry& e : x->entries)
    if (e.live && --x->pool->rc[e.block] == 0) x->pool->free_ids.insert(e.block);
  delete x;
}

zp_status zp_prefix_insert(zp_prefix_index* x, const int32_t* tokens, int32_t num_tokens,
                           const int32_t* block_ids, int32_t num_blocks, int32_t* num_added) {
  zp::clear_error();
  if (!x || (num_tokens > 0 && !tokens) || (num_blocks > 0 && !block_ids)) {
    zp::set_error("NULL argument");
    return ZP_ERR_INVALID;
  }
  const int32_t full = std::min(num_tokens / x->b, num_blocks);
  for (int32_t n = 0; n < full; n++) {
    const int32_t id = block_ids[n];
    if (id < 0 || id >= x->pool->num_blocks || x->pool->rc[id] < 1) {
      zp::set_error("block %d (position %d) is not an allocated block", id, n);
      return ZP_ERR_INVALID;
    }
  }
  int32_t parent = -1, added = 0;
  x->clock++;
  for (int32_t n = 0; n < full; n++) {
    const int32_t* tk = tokens + (size_t)n * x->b;
    int32_t e = x->find(parent, tk);
    if (e < 0) {
      if (!x->free_entries.empty()) {
        e = x->free_entries.back();
        x->free_entries.pop_back();
      } else {
        e = (int32_t)x->entries.size();
        x->entries.emplace_back();
      }
      Entry& ne = x->entries[(size_t)e];
      ne.parent = parent;
      ne.block = block_ids[n];
      ne.children = 0;
      ne.live = true;
      ne.tokens.assign(tk, tk + x->b);
      x->pool->rc[ne.block] += 1;  // the index's reference
      if (parent >= 0) x->entries[(size_t)parent].children++;
      x->by_key.emplace(key_of(parent, tk, x->b), e);
      x->live++;
      added++;
    }
    x->entries[(size_t)e].last_used = x->clock;
    parent = e;
  }
  if (num_added) *num_added = added;
  return ZP_OK;
}

zp_status zp_prefix_match(zp_prefix_index* x, const int32_t* tokens, int32_t num_tokens,
                          int32_t* block_ids_out, int32_t* num_matched) {
  zp::clear_error();
  if (!x || !num_matched || (num_tokens > 0 && (!tokens || !block_ids_out))) {
    zp::set_error("NULL argument");
    return ZP_ERR_INVALID;
  }
  if (x->pool->poisoned) { zp::set_error("pool unusable after an earlier HIP failure"); return ZP_ERR_STATE; }
  int32_t parent = -1, n = 0;
  x->clock++;
  for (; n < num_tokens / x->b; n++) {
    const int32_t e = x->find(parent, tokens + (size_t)n * x->b);
    if (e < 0) break;
    x->entries[(size_t)e].last_used = x->clock;
    block_ids_out[n] = x->entries[(size_t)e].block;
    x->pool->rc[x->entries[(size_t)e].block] += 1;  // the caller's reference
    parent = e;
  }
  *num_matched = n;
  return ZP_OK;
}

zp_status zp_prefix_evict(zp_prefix_index* x, int32_t max_entries, int32_t* freed_out,
                          int32_t* num_freed) {
  zp::clear_error();
  if (!x || max_entries < 0) { zp::set_error("bad argument"); return ZP_ERR_INVALID; }
  int32_t dropped = 0, freed = 0;
  while (dropped < max_entries) {
    // least recently used entry without children (a leaf of the prefix tree)
    int32_t best = -1;
    for (int32_t i = 0; i < (int32_t)x->entries.size(); i++) {
      const Entry& e = x->entries[(size_t)i];
      if (e.live && e.children == 0 &&
          (best < 0 || e.last_used < x->entries[(size_t)best].last_used))
        best = i;
    }
    if (best < 0) break;
    Entry& e = x->entries[(size_t)best];
    auto range = x->by_key.equal_range(key_of(e.parent, e.tokens.data(), x->b));
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == best) {
        x->by_key.erase(it);
        break;
      }
    if (e.parent >= 0) x->entries[(size_t)e.parent].children--;
    if (--x->pool->rc[e.block] == 0) {
      x->pool->free_ids.insert(e.block);
      if (freed_out) freed_out[freed] = e.block;
      freed++;
    }
    e.live = false;
    e.tokens.clear();
    x->free_entries.push_back(best);
    x->live--;
    dropped++;
  }
  if (num_freed) *num_freed = freed;
  return ZP_OK;
}

int32_t zp_prefix_size(const zp_prefix_index* x) { return x ? x->live : -1; }

}  // extern "C"
