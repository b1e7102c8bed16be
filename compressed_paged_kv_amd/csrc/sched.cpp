// Hybrid scheduler of a Compressed PagedAttention engine (host C++).
//
// Requests below the block cap decode without any extra resource; only a
// request that is about to need compression holds a query slot (storage for
// the queries of its last w tokens, the observation window); when blocks
// run out, requests are preempted, those without a query slot first (nl
// page "Technische samenvatting", Methodologie item 2; ko page "기술 요약",
// section 2.B).  Block tables and counts live in the block pool; a request
// at the cap is handed to the compression call, whose planner rewrites its
// table (nl page Methodologie item 1).
//
// One plan per engine step.  For every running request, in admission order:
//   * at the cap (seq_len = N_max*b): it compresses this step and decodes
//     again from the next one (the asynchronous scheme of the ko page,
//     section 2.D: the other requests do not wait for it);
//   * otherwise it decodes one token at position p = seq_len: a new block
//     when p starts one it does not hold (after a compression the reserved
//     block is already there); a query slot when p lies in the window
//     [N_max*b - w, N_max*b) -- free slots go to the requests that have
//     waited longest (then the earliest admitted), the others wait this
//     step; the query of position p goes to row slot*w + (p - (N_max*b - w)).
// Block shortage: blocks given back in a step (by finished or preempted
// requests) become allocatable only after the fence, so a request that
// finds no free block waits for the step; unless blocks given back earlier
// in the step already cover it, it also preempts the running request
// without a query slot that was admitted last (then, if none, the one with
// a slot admitted last; possibly itself), never one compressing this step.
// A preempted request gives back its blocks and slot and returns to the
// front of the queue to start over.
// Chunked prefill (config prefill_chunk > 0): a prompt is written chunk by
// chunk, one chunk per step, so a prompt longer than the budget never holds
// more than a chunk beyond it (the ko page, section 5, names chunked
// prefilling as the next step; the nl page's problem statement faults
// compressing only the input for the prefill cost it leaves).  Between steps
// a prefilling request's cache ends at or below the window start T - w
// (T = N_max*b).  The next chunk, of c = min(prefill_chunk, rest) prompt
// tokens from cache position t:
//   * ends at or below T - w: written as it is;
//   * else, if the rest of the prompt reaches T: cut (or stretched) to end
//     at the block boundary max(T, floor((t + c)/b)*b) and compressed in the
//     same step, n_src = that boundary / b blocks (zp_compress_n, the window
//     being the chunk's last w queries); the cache is then back to
//     (N_max-1)*b <= T - w;
//   * else the rest ends inside the window band (T - w, T): it is written
//     whole, its positions at or past T - w recorded in a query slot (the
//     request waits for one like a decoding request), and decode continues.
// Then waiting requests are admitted in order while their prompt blocks (the
// first chunk's, with chunked prefill) and the concurrency cap allow.
// Blocks given back are released to the pool as a pending group (reference
// count 0, not allocatable) that the caller releases with
// zp_block_pool_fence once the GPU work of the step has completed.
#include <algorithm>
#include <cstring>
#include <deque>
#include <set>
#include <unordered_map>
#include <vector>

#include "block_pool.h"
#include "zp_internal.h"

namespace {

struct Req {
  int64_t id = 0;
  int32_t prompt_len = 0, max_new = 0, generated = 0;
  int32_t seq_len = 0;
  int32_t prompt_done = 0;       // prompt tokens written (chunked prefill)
  int32_t compress_n_src = 0;    // blocks held by a request compressing this step
  std::vector<int32_t> table;
  int32_t qslot = -1;
  int64_t admit_order = -1;
  int64_t slot_wait_since = -1;  // step since which it waits for a query slot
  bool running = false;
  bool compress_now = false;
  bool done = false;
};

}  // namespace

struct zp_sched {
  zp_block_pool* pool = nullptr;
  zp_sched_config cfg{};
  std::unordered_map<int64_t, Req> reqs;
  std::deque<int64_t> waiting;
  std::vector<int64_t> running;  // admission order
  std::set<int32_t> free_qslots;
  int64_t admit_counter = 0;
  int64_t step = 0;
  // outputs of the last plan
  std::vector<int64_t> admitted, decode_ids, compress_ids, preempted, finished, prefill_ids;
  std::vector<int32_t> decode_slot, decode_seq, decode_row, compress_qslot, compress_n_src;
  std::vector<int32_t> prefill_start, prefill_len, prefill_row;
  std::vector<int32_t> to_release;
};

namespace {

int32_t cap_tokens(const zp_sched* s) { return s->cfg.n_max * s->cfg.block_size; }

bool prefilling(const Req& q) { return q.prompt_done < q.prompt_len; }

// Length of the next prefill chunk of q (cache at t = q.seq_len, t <= T - w)
// and whether the request compresses right after it (see the header).
int32_t next_chunk(const zp_sched* s, const Req& q, bool* compress) {
  const int32_t b = s->cfg.block_size, w = s->cfg.window, T = cap_tokens(s);
  const int32_t t = q.seq_len, rest = q.prompt_len - q.prompt_done;
  const int32_t c = std::min(s->cfg.prefill_chunk, rest);
  *compress = false;
  if (t + c <= T - w) return c;
  if (t + rest >= T) {
    *compress = true;
    return std::max(T, (t + c) / b * b) - t;
  }
  return rest;
}

// Drop a request's references to its blocks; blocks reaching 0 wait in the
// pool for zp_block_pool_fence.
void give_back_blocks(zp_sched* s, Req& q) {
  for (int32_t id : q.table) {
    if (--s->pool->rc[id] == 0) s->to_release.push_back(id);
  }
  q.table.clear();
  if (q.qslot >= 0) {
    s->free_qslots.insert(q.qslot);
    q.qslot = -1;
  }
}

bool alloc_block(zp_sched* s, int32_t* id) {
  s->pool->reap();
  if (s->pool->free_ids.empty()) return false;
  *id = *s->pool->free_ids.begin();
  s->pool->free_ids.erase(s->pool->free_ids.begin());
  s->pool->rc[*id] = 1;
  return true;
}

// The victim for a block shortage: among running requests that are not
// compressing this step (and, if `exclude` >= 0, not that one), the last
// admitted without a query slot, else the last admitted with one.
int64_t pick_victim(zp_sched* s, int64_t exclude) {
  int64_t best = -1;
  int best_rank = -1;
  int64_t best_order = -1;
  for (int64_t id : s->running) {
    const Req& q = s->reqs[id];
    if (q.compress_now || id == exclude) continue;
    const int rank = q.qslot < 0 ? 1 : 0;
    if (rank > best_rank || (rank == best_rank && q.admit_order > best_order)) {
      best = id;
      best_rank = rank;
      best_order = q.admit_order;
    }
  }
  return best;
}

void preempt(zp_sched* s, int64_t id) {
  Req& q = s->reqs[id];
  give_back_blocks(s, q);
  q.running = false;
  q.seq_len = 0;
  q.prompt_done = 0;
  q.generated = 0;
  q.admit_order = -1;
  q.slot_wait_since = -1;
  s->running.erase(std::find(s->running.begin(), s->running.end(), id));
  s->waiting.push_front(id);
  s->preempted.push_back(id);
}

}  // namespace

extern "C" {

zp_status zp_sched_create(zp_block_pool* pool, const zp_sched_config* cfg, zp_sched** out) {
  zp::clear_error();
  if (!pool || !cfg || !out) { zp::set_error("pool, cfg and out must not be NULL"); return ZP_ERR_INVALID; }
  if (cfg->n_max < 2 || (cfg->block_size != 16 && cfg->block_size != 32) || cfg->window < 1 ||
      cfg->window > cfg->block_size || cfg->num_query_slots < 1 || cfg->max_running < 1) {
    zp::set_error("bad config: n_max >= 2, block_size in {16,32}, 1 <= window <= block_size, "
                  "num_query_slots >= 1, max_running >= 1");
    return ZP_ERR_INVALID;
  }
  // a chunk spans at most prefill_chunk + b tokens past the cache (the
  // stretch to the next block boundary), so its compression holds at most
  // n_max - 1 + prefill_chunk/b + 1 blocks and evicts at most
  // prefill_chunk + 2b slots per head
  if (cfg->prefill_chunk < 0 || cfg->prefill_chunk % cfg->block_size != 0 ||
      (cfg->prefill_chunk > 0 &&
       (cfg->n_max + cfg->prefill_chunk / cfg->block_size > zp::kMaxCompressBlocks ||
        (int64_t)(cfg->n_max + cfg->prefill_chunk / cfg->block_size) * cfg->block_size >
            zp::kMaxScoreSlots ||
        cfg->prefill_chunk + 2 * cfg->block_size > zp::kMaxEvicted))) {
    zp::set_error("prefill_chunk %d: a multiple of block_size, with n_max + prefill_chunk/b <= %d "
                  "blocks of at most %d tokens and prefill_chunk + 2*block_size <= %d",
                  cfg->prefill_chunk, zp::kMaxCompressBlocks, zp::kMaxScoreSlots, zp::kMaxEvicted);
    return ZP_ERR_INVALID;
  }
  zp_sched* s = new zp_sched();
  s->pool = pool;
  s->cfg = *cfg;
  for (int32_t i = 0; i < cfg->num_query_slots; i++) s->free_qslots.insert(i);
  *out = s;
  return ZP_OK;
}

void zp_sched_destroy(zp_sched* s) { delete s; }

zp_status zp_sched_add(zp_sched* s, int64_t id, int32_t prompt_len, int32_t max_new_tokens) {
  zp::clear_error();
  if (!s) { zp::set_error("scheduler is NULL"); return ZP_ERR_INVALID; }
  if (s->reqs.count(id)) { zp::set_error("request %lld already exists", (long long)id); return ZP_ERR_INVALID; }
  if (s->cfg.prefill_chunk == 0 &&
      (prompt_len < 1 || prompt_len > cap_tokens(s) - s->cfg.window || max_new_tokens < 1)) {
    zp::set_error("prompt_len must be in [1, N_max*b - w = %d] and max_new_tokens >= 1 (longer "
                  "prompts need prefill_chunk > 0)", cap_tokens(s) - s->cfg.window);
    return ZP_ERR_INVALID;
  }
  if (prompt_len < 1 || max_new_tokens < 1) {
    zp::set_error("prompt_len and max_new_tokens must be >= 1");
    return ZP_ERR_INVALID;
  }
  Req q;
  q.id = id;
  q.prompt_len = prompt_len;
  q.max_new = max_new_tokens;
  s->reqs[id] = q;
  s->waiting.push_back(id);
  return ZP_OK;
}

zp_status zp_sched_plan(zp_sched* s, zp_sched_step* out) {
  zp::clear_error();
  if (!s || !out) { zp::set_error("scheduler and out must not be NULL"); return ZP_ERR_INVALID; }
  if (s->pool->poisoned) { zp::set_error("pool unusable after an earlier HIP failure"); return ZP_ERR_STATE; }
  for (int64_t id : s->compress_ids) {
    if (s->reqs.count(id) && s->reqs[id].compress_now) {
      zp::set_error("request %lld was planned to compress but zp_sched_compress_commit was not called",
                    (long long)id);
      return ZP_ERR_STATE;
    }
  }
  const int32_t b = s->cfg.block_size, w = s->cfg.window, T = cap_tokens(s);
  s->admitted.clear();
  s->decode_ids.clear();
  s->decode_slot.clear();
  s->decode_seq.clear();
  s->decode_row.clear();
  s->compress_ids.clear();
  s->compress_qslot.clear();
  s->compress_n_src.clear();
  s->prefill_ids.clear();
  s->prefill_start.clear();
  s->prefill_len.clear();
  s->prefill_row.clear();
  s->preempted.clear();
  s->finished.clear();
  s->to_release.clear();

  // 1. requests that produced their last token in the previous step finish
  for (size_t i = 0; i < s->running.size();) {
    Req& q = s->reqs[s->running[i]];
    if (q.generated >= q.max_new) {
      give_back_blocks(s, q);
      q.running = false;
      q.done = true;
      s->finished.push_back(q.id);
      s->running.erase(s->running.begin() + (long)i);
    } else {
      i++;
    }
  }

  // 2a. the requests at the cap compress; requests whose next token is in
  //     the window need a query slot: free slots go to them in the order they
  //     started waiting (then admission order), the others wait this step
  std::vector<int64_t> need_slot;
  for (int64_t id : s->running) {
    Req& q = s->reqs[id];
    if (prefilling(q)) continue;  // chunks are planned in 2c
    if (q.seq_len == T) {
      q.compress_now = true;
      q.compress_n_src = s->cfg.n_max;
      s->compress_ids.push_back(id);
    } else if (q.seq_len >= T - w && q.qslot < 0) {
      if (q.slot_wait_since < 0) q.slot_wait_since = s->step;
      need_slot.push_back(id);
    }
  }
  std::stable_sort(need_slot.begin(), need_slot.end(), [&](int64_t a, int64_t c) {
    return s->reqs[a].slot_wait_since < s->reqs[c].slot_wait_since;
  });
  for (int64_t id : need_slot) {
    if (s->free_qslots.empty()) break;
    Req& q = s->reqs[id];
    q.qslot = *s->free_qslots.begin();
    s->free_qslots.erase(s->free_qslots.begin());
    q.slot_wait_since = -1;
  }
  std::vector<int64_t> order;
  for (int64_t id : s->running) {
    const Req& q = s->reqs[id];
    if (prefilling(q) || q.compress_now || (q.seq_len >= T - w && q.qslot < 0)) continue;
    order.push_back(id);
  }
  // 2b. in admission order: one token each, a new block when it starts one
  int64_t promised = (int64_t)s->to_release.size();  // given back, allocatable after the fence
  for (int64_t id : order) {
    if (!s->reqs[id].running) continue;  // preempted earlier in this step
    Req& q = s->reqs[id];
    const int32_t p = q.seq_len;
    if (p / b >= (int32_t)q.table.size()) {  // p starts a block it does not hold yet
      int32_t blk = -1;
      if (!alloc_block(s, &blk)) {
        // Blocks given back in this step only become allocatable after the
        // fence, so the request waits; it preempts a victim unless blocks
        // already given back in this step cover it.
        if (promised > 0) {
          promised--;
          continue;
        }
        const int64_t v = pick_victim(s, -1);
        if (v < 0) {
          zp::set_error("request %lld needs a block and none can be freed", (long long)id);
          return ZP_ERR_NO_BLOCKS;
        }
        // a victim already planned to decode this step drops out of the plan
        auto it = std::find(s->decode_ids.begin(), s->decode_ids.end(), v);
        if (it != s->decode_ids.end()) {
          const size_t k = (size_t)(it - s->decode_ids.begin());
          s->decode_ids.erase(it);
          s->decode_slot.erase(s->decode_slot.begin() + (long)k);
          s->decode_seq.erase(s->decode_seq.begin() + (long)k);
          s->decode_row.erase(s->decode_row.begin() + (long)k);
        }
        const size_t before = s->to_release.size();
        preempt(s, v);
        promised += (int64_t)(s->to_release.size() - before) - (v != id ? 1 : 0);
        continue;
      }
      q.table.push_back(blk);
    }
    const bool window = p >= T - w;
    s->decode_ids.push_back(id);
    s->decode_slot.push_back(q.table[(size_t)(p / b)] * b + p % b);
    s->decode_seq.push_back(p + 1);
    s->decode_row.push_back(window ? q.qslot * w + (p - (T - w)) : -1);
    q.seq_len = p + 1;
    q.generated += 1;
  }
  // 2c. chunked prefill, in admission order: one chunk each (see the header)
  std::vector<int64_t> pre;
  for (int64_t id : s->running)
    if (prefilling(s->reqs[id])) pre.push_back(id);
  for (int64_t id : pre) {
    if (!s->reqs[id].running) continue;  // preempted earlier in this step
    Req& q = s->reqs[id];
    bool comp = false;
    const int32_t c = next_chunk(s, q, &comp);
    const int32_t t = q.seq_len;
    const bool band = !comp && t + c > T - w;  // ends inside the window band
    if (band && q.qslot < 0) {
      if (s->free_qslots.empty()) continue;  // waits for a query slot
      q.qslot = *s->free_qslots.begin();
      s->free_qslots.erase(s->free_qslots.begin());
    }
    const int32_t need = (t + c + b - 1) / b - (int32_t)q.table.size();
    s->pool->reap();
    if (need > (int32_t)s->pool->free_ids.size()) {
      // as for a decoding request: wait, and preempt unless blocks given
      // back in this step cover it
      if (promised >= need) {
        promised -= need;
        continue;
      }
      const int64_t v = pick_victim(s, -1);
      if (v < 0) {
        zp::set_error("request %lld needs %d blocks and none can be freed", (long long)id, need);
        return ZP_ERR_NO_BLOCKS;
      }
      auto it = std::find(s->decode_ids.begin(), s->decode_ids.end(), v);
      if (it != s->decode_ids.end()) {
        const size_t k = (size_t)(it - s->decode_ids.begin());
        s->decode_ids.erase(it);
        s->decode_slot.erase(s->decode_slot.begin() + (long)k);
        s->decode_seq.erase(s->decode_seq.begin() + (long)k);
        s->decode_row.erase(s->decode_row.begin() + (long)k);
      }
      auto jt = std::find(s->prefill_ids.begin(), s->prefill_ids.end(), v);
      if (jt != s->prefill_ids.end()) {
        const size_t k = (size_t)(jt - s->prefill_ids.begin());
        s->prefill_ids.erase(jt);
        s->prefill_start.erase(s->prefill_start.begin() + (long)k);
        s->prefill_len.erase(s->prefill_len.begin() + (long)k);
        s->prefill_row.erase(s->prefill_row.begin() + (long)k);
      }
      const size_t before = s->to_release.size();
      preempt(s, v);
      promised += (int64_t)(s->to_release.size() - before);
      continue;
    }
    for (int32_t i = 0; i < need; i++) {
      int32_t blk = -1;
      alloc_block(s, &blk);
      q.table.push_back(blk);
    }
    s->prefill_ids.push_back(id);
    s->prefill_start.push_back(t);
    s->prefill_len.push_back(c);
    s->prefill_row.push_back(band ? q.qslot * w : -1);
    q.seq_len = t + c;
    q.prompt_done += c;
    if (comp) {
      q.compress_now = true;
      q.compress_n_src = (t + c) / b;
      s->compress_ids.push_back(id);
    }
  }

  // 3. admission in arrival order, while the prompt blocks (with chunked
  //    prefill: the first chunk's) fit; a chunked request's first chunk is
  //    written in this step
  while (!s->waiting.empty() && (int32_t)s->running.size() < s->cfg.max_running) {
    Req& q = s->reqs[s->waiting.front()];
    const bool chunked = s->cfg.prefill_chunk > 0;
    bool comp = false;
    q.seq_len = 0;
    q.prompt_done = 0;
    const int32_t c = chunked ? next_chunk(s, q, &comp) : q.prompt_len;
    const bool band = chunked && !comp && c > T - w;
    const int32_t nb = (c + b - 1) / b;
    s->pool->reap();
    if ((int32_t)s->pool->free_ids.size() < nb || (band && s->free_qslots.empty())) break;
    s->waiting.pop_front();
    for (int32_t i = 0; i < nb; i++) {
      int32_t blk = -1;
      alloc_block(s, &blk);
      q.table.push_back(blk);
    }
    q.seq_len = c;
    q.prompt_done = c;
    q.generated = 0;
    q.running = true;
    q.admit_order = s->admit_counter++;
    s->running.push_back(q.id);
    s->admitted.push_back(q.id);
    if (chunked) {
      if (band) {
        q.qslot = *s->free_qslots.begin();
        s->free_qslots.erase(s->free_qslots.begin());
      }
      s->prefill_ids.push_back(q.id);
      s->prefill_start.push_back(0);
      s->prefill_len.push_back(c);
      s->prefill_row.push_back(band ? q.qslot * w : -1);
      if (comp) {
        q.compress_now = true;
        q.compress_n_src = c / b;
        s->compress_ids.push_back(q.id);
      }
    }
  }
  for (int64_t id : s->compress_ids) {
    s->compress_qslot.push_back(s->reqs[id].qslot);
    s->compress_n_src.push_back(s->reqs[id].compress_n_src);
  }
  // decodes longest first: the paged decode dispatches its workgroups in
  // request order, and a ragged batch finishes sooner when its long requests
  // start first (equal lengths keep their order)
  {
    const size_t nd = s->decode_ids.size();
    std::vector<size_t> order(nd);
    for (size_t i = 0; i < nd; i++) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](size_t a, size_t c) { return s->decode_seq[a] > s->decode_seq[c]; });
    auto permute = [&](auto& v) {
      auto old = v;
      for (size_t i = 0; i < nd; i++) v[i] = old[order[i]];
    };
    permute(s->decode_ids);
    permute(s->decode_slot);
    permute(s->decode_seq);
    permute(s->decode_row);
  }
  zp::add_pending(s->pool, s->to_release, nullptr);
  s->step++;

  out->num_admitted = (int32_t)s->admitted.size();
  out->admitted = s->admitted.data();
  out->num_decode = (int32_t)s->decode_ids.size();
  out->decode_ids = s->decode_ids.data();
  out->decode_slot = s->decode_slot.data();
  out->decode_seq_len = s->decode_seq.data();
  out->decode_record_row = s->decode_row.data();
  out->num_compress = (int32_t)s->compress_ids.size();
  out->compress_ids = s->compress_ids.data();
  out->compress_qslot = s->compress_qslot.data();
  out->compress_n_src = s->compress_n_src.data();
  out->num_prefill = (int32_t)s->prefill_ids.size();
  out->prefill_ids = s->prefill_ids.data();
  out->prefill_start = s->prefill_start.data();
  out->prefill_len = s->prefill_len.data();
  out->prefill_record_row = s->prefill_row.data();
  out->num_preempted = (int32_t)s->preempted.size();
  out->preempted = s->preempted.data();
  out->num_finished = (int32_t)s->finished.size();
  out->finished = s->finished.data();
  out->num_released = (int32_t)s->to_release.size();
  return ZP_OK;
}

zp_status zp_sched_tables(const zp_sched* s, const int64_t* ids, int32_t n, int32_t width,
                          int32_t* tables_out, int32_t* seq_lens_out) {
  zp::clear_error();
  if (!s || (n > 0 && (!ids || !tables_out))) { zp::set_error("NULL argument"); return ZP_ERR_INVALID; }
  if (width < s->cfg.n_max) { zp::set_error("width %d below n_max %d", width, s->cfg.n_max); return ZP_ERR_INVALID; }
  for (int32_t i = 0; i < n; i++) {
    auto it = s->reqs.find(ids[i]);
    if (it == s->reqs.end()) { zp::set_error("unknown request %lld", (long long)ids[i]); return ZP_ERR_INVALID; }
    const Req& q = it->second;
    int32_t* row = tables_out + (size_t)i * width;
    for (int32_t k = 0; k < width; k++) row[k] = k < (int32_t)q.table.size() ? q.table[(size_t)k] : -1;
    if (seq_lens_out) seq_lens_out[i] = q.seq_len;
  }
  return ZP_OK;
}

zp_status zp_sched_compress_commit(zp_sched* s, const int32_t* new_tables) {
  zp::clear_error();
  if (!s) { zp::set_error("scheduler is NULL"); return ZP_ERR_INVALID; }
  if (!s->compress_ids.empty() && !new_tables) { zp::set_error("new_tables is NULL"); return ZP_ERR_INVALID; }
  const int32_t n_max = s->cfg.n_max, K_keep = (n_max - 1) * s->cfg.block_size;
  for (size_t i = 0; i < s->compress_ids.size(); i++) {
    Req& q = s->reqs[s->compress_ids[i]];
    if (!q.compress_now) continue;
    q.table.assign(new_tables + i * (size_t)n_max, new_tables + (i + 1) * (size_t)n_max);
    q.seq_len = K_keep;
    q.compress_now = false;
    if (q.qslot >= 0) {
      s->free_qslots.insert(q.qslot);
      q.qslot = -1;
    }
  }
  return ZP_OK;
}

zp_status zp_sched_stats(const zp_sched* s, int32_t* num_waiting, int32_t* num_running,
                         int32_t* free_query_slots) {
  zp::clear_error();
  if (!s) { zp::set_error("scheduler is NULL"); return ZP_ERR_INVALID; }
  if (num_waiting) *num_waiting = (int32_t)s->waiting.size();
  if (num_running) *num_running = (int32_t)s->running.size();
  if (free_query_slots) *free_query_slots = (int32_t)s->free_qslots.size();
  return ZP_OK;
}

}  // extern "C"
