// Block pool and compression planner (host C++).
//
// Reference counts and allocate-then-decrement sharing follow the paged
// cache guide at upskillscore.com ("How it works"); new target blocks for
// shared blocks follow the Zipage summaries (ko page, "기술 요약" section
// 2.C; nl page, "Technische samenvatting", Methodologie item 3); the trigger,
// the N_max-1 target blocks and the reserved last block follow nl page
// Methodologie item 1 and ko page section 2.A.
#include "block_pool.h"

#include <algorithm>
#include <cstring>

#include "zp_internal.h"

void zp_block_pool::reap() {
  size_t keep = 0;
  for (size_t i = 0; i < pending.size(); i++) {
    Pending& p = pending[i];
    bool done = false;
    if (p.event != nullptr) {
      hipError_t e = hipEventQuery(p.event);
      if (e == hipSuccess) {
        done = true;
      } else if (e != hipErrorNotReady) {
        poisoned = true;  // the GPU work failed; its blocks can never be trusted
      }
    }
    if (done) {
      for (int32_t id : p.ids) free_ids.insert(id);
      give_back_event(p.event);
    } else {
      if (keep != i) pending[keep] = std::move(p);
      keep++;
    }
  }
  pending.resize(keep);
}

hipError_t zp_block_pool::take_event(hipEvent_t* out) {
  if (!spare_events.empty()) {
    *out = spare_events.back();
    spare_events.pop_back();
    return hipSuccess;
  }
  return hipEventCreateWithFlags(out, hipEventDisableTiming);
}

void zp_block_pool::give_back_event(hipEvent_t e) {
  if (e) spare_events.push_back(e);
}

int32_t zp_block_pool::pending_count() const {
  int64_t n = 0;
  for (const Pending& p : pending) n += (int64_t)p.ids.size();
  return (int32_t)n;
}

namespace zp {

void add_pending(zp_block_pool* pool, std::vector<int32_t> ids, hipEvent_t event) {
  if (ids.empty()) {
    pool->give_back_event(event);
    return;
  }
  zp_block_pool::Pending p;
  p.event = event;
  p.ids = std::move(ids);
  pool->pending.push_back(std::move(p));
}

zp_status plan_compression(zp_block_pool* pool, int32_t n_src, int32_t n_max, int32_t num_reqs,
                           int32_t* block_tables, PlanResult* out, const int32_t* first_evict,
                           int32_t block_size, bool dry_run, const int32_t* num_blocks) {
  // shared block n of request r that stays: every slot of it lies below the
  // request's first eviction in every layer and head
  auto kept_shared = [&](int32_t r, int32_t n) {
    return first_evict && n < n_max - 1 && (int64_t)(n + 1) * block_size <= first_evict[r];
  };
  if (!pool) { set_error("pool is NULL"); return ZP_ERR_INVALID; }
  if (pool->poisoned) { set_error("pool unusable after an earlier HIP failure"); return ZP_ERR_STATE; }
  if (n_max < 2) { set_error("n_max must be >= 2 (got %d)", n_max); return ZP_ERR_INVALID; }
  if (n_src < n_max) { set_error("n_src (%d) must be >= n_max (%d)", n_src, n_max); return ZP_ERR_INVALID; }
  if (num_reqs < 0) { set_error("num_reqs < 0"); return ZP_ERR_INVALID; }
  if (num_reqs > 0 && !block_tables) { set_error("block_tables is NULL"); return ZP_ERR_INVALID; }
  // blocks request r holds: num_blocks[r] (the rest of its row is -1), or n_src
  auto held = [&](int32_t r) { return num_blocks ? num_blocks[r] : n_src; };
  if (num_blocks)
    for (int32_t r = 0; r < num_reqs; r++) {
      if (num_blocks[r] < n_max || num_blocks[r] > n_src) {
        set_error("request %d holds %d blocks, not in [n_max=%d, n_src=%d]", r, num_blocks[r],
                  n_max, n_src);
        return ZP_ERR_INVALID;
      }
      for (int32_t n = num_blocks[r]; n < n_src; n++)
        if (block_tables[(size_t)r * n_src + n] != -1) {
          set_error("request %d: entry %d past its %d blocks is not -1", r, n, num_blocks[r]);
          return ZP_ERR_INVALID;
        }
    }
  const int32_t nb = pool->num_blocks;
  const std::vector<int32_t>& rc0 = pool->rc;  // counts at the start of the call
  std::vector<int32_t> seen(nb, 0);
  std::vector<int32_t> last_row(nb, -1);  // last request whose table held the id
  int64_t need = 0;
  for (int32_t r = 0; r < num_reqs; r++) {
    const int32_t* row = block_tables + (size_t)r * n_src;
    for (int32_t n = 0; n < held(r); n++) {
      const int32_t id = row[n];
      if (id < 0 || id >= nb) {
        set_error("request %d block %d: id %d out of range [0, %d)", r, n, id, nb);
        return ZP_ERR_INVALID;
      }
      if (rc0[id] < 1) {
        set_error("request %d block %d: id %d is not allocated", r, n, id);
        return ZP_ERR_INVALID;
      }
      if (last_row[id] == r) {
        set_error("request %d: id %d appears twice in its table", r, id);
        return ZP_ERR_INVALID;
      }
      last_row[id] = r;
      if (++seen[id] > rc0[id]) {
        set_error("id %d listed %d times but its refcount is %d", id, seen[id], rc0[id]);
        return ZP_ERR_INVALID;
      }
      if (n < n_max && rc0[id] > 1 && !kept_shared(r, n)) need++;
    }
  }
  if (dry_run) return ZP_OK;  // the tables are valid; the block count is checked later
  pool->reap();
  if (need > (int64_t)pool->free_ids.size()) {
    set_error("need %lld new target blocks, %zu free", (long long)need, pool->free_ids.size());
    return ZP_ERR_NO_BLOCKS;
  }

  // Commit.  Decisions use the counts from the start of the call, so two
  // requests sharing a block both re-target it and the last one frees it.
  // Blocks n_max.. are surplus (nl page Methodologie item 1: released).
  const std::vector<int32_t> start_rc = rc0;
  out->src.assign(block_tables, block_tables + (size_t)num_reqs * n_src);
  out->dst.assign((size_t)num_reqs * (n_max - 1), 0);
  out->freed.clear();
  for (int32_t r = 0; r < num_reqs; r++) {
    int32_t* row = block_tables + (size_t)r * n_src;
    for (int32_t n = 0; n < held(r); n++) {
      const int32_t s = row[n];
      if (n >= n_max) {
        if (--pool->rc[s] == 0) out->freed.push_back(s);
        row[n] = -1;
        continue;
      }
      int32_t target = s;
      if (start_rc[s] > 1 && !kept_shared(r, n)) {
        target = *pool->free_ids.begin();
        pool->free_ids.erase(pool->free_ids.begin());
        pool->rc[target] = 1;
        if (--pool->rc[s] == 0) out->freed.push_back(s);
      }
      if (n < n_max - 1) out->dst[(size_t)r * (n_max - 1) + n] = target;
      row[n] = target;
    }
  }
  return ZP_OK;
}

}  // namespace zp

extern "C" {

zp_status zp_block_pool_create(int32_t num_blocks, uint32_t flags, zp_block_pool** out) {
  zp::clear_error();
  if (!out) { zp::set_error("out is NULL"); return ZP_ERR_INVALID; }
  if (num_blocks <= 0) { zp::set_error("num_blocks must be > 0"); return ZP_ERR_INVALID; }
  if (flags & ~ZP_POOL_MANUAL_FENCE) { zp::set_error("unknown flags 0x%x", flags); return ZP_ERR_INVALID; }
  zp_block_pool* p = new zp_block_pool();
  p->num_blocks = num_blocks;
  p->flags = flags;
  p->rc.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; i++) p->free_ids.insert(p->free_ids.end(), i);
  *out = p;
  return ZP_OK;
}

void zp_block_pool_destroy(zp_block_pool* pool) {
  if (!pool) return;
  for (auto& p : pool->pending)
    if (p.event) {
      (void)hipEventSynchronize(p.event);
      (void)hipEventDestroy(p.event);
    }
  for (hipEvent_t e : pool->spare_events) (void)hipEventDestroy(e);
  delete pool;
}

zp_status zp_block_alloc(zp_block_pool* pool, int32_t n, int32_t* ids_out) {
  zp::clear_error();
  if (!pool) { zp::set_error("pool is NULL"); return ZP_ERR_INVALID; }
  if (pool->poisoned) { zp::set_error("pool unusable after an earlier HIP failure"); return ZP_ERR_STATE; }
  if (n < 0 || (n > 0 && !ids_out)) { zp::set_error("bad n or ids_out"); return ZP_ERR_INVALID; }
  pool->reap();
  if ((size_t)n > pool->free_ids.size()) {
    zp::set_error("asked for %d blocks, %zu free", n, pool->free_ids.size());
    return ZP_ERR_NO_BLOCKS;
  }
  for (int32_t i = 0; i < n; i++) {
    const int32_t id = *pool->free_ids.begin();
    pool->free_ids.erase(pool->free_ids.begin());
    pool->rc[id] = 1;
    ids_out[i] = id;
  }
  return ZP_OK;
}

zp_status zp_block_share(zp_block_pool* pool, const int32_t* ids, int32_t n) {
  zp::clear_error();
  if (!pool) { zp::set_error("pool is NULL"); return ZP_ERR_INVALID; }
  if (pool->poisoned) { zp::set_error("pool unusable after an earlier HIP failure"); return ZP_ERR_STATE; }
  if (n < 0 || (n > 0 && !ids)) { zp::set_error("bad n or ids"); return ZP_ERR_INVALID; }
  for (int32_t i = 0; i < n; i++)
    if (ids[i] < 0 || ids[i] >= pool->num_blocks || pool->rc[ids[i]] < 1) {
      zp::set_error("id %d is not an allocated block", ids[i]);
      return ZP_ERR_INVALID;
    }
  for (int32_t i = 0; i < n; i++) pool->rc[ids[i]] += 1;
  return ZP_OK;
}

zp_status zp_block_release(zp_block_pool* pool, const int32_t* ids, int32_t n, int32_t* freed_out,
                           int32_t* n_freed) {
  zp::clear_error();
  if (!pool) { zp::set_error("pool is NULL"); return ZP_ERR_INVALID; }
  if (pool->poisoned) { zp::set_error("pool unusable after an earlier HIP failure"); return ZP_ERR_STATE; }
  if (n < 0 || (n > 0 && !ids)) { zp::set_error("bad n or ids"); return ZP_ERR_INVALID; }
  // validate against the counts this call would reach (an id may repeat)
  std::vector<std::pair<int32_t, int32_t>> dec;
  for (int32_t i = 0; i < n; i++) {
    if (ids[i] < 0 || ids[i] >= pool->num_blocks) {
      zp::set_error("id %d out of range", ids[i]);
      return ZP_ERR_INVALID;
    }
    dec.emplace_back(ids[i], 1);
  }
  std::sort(dec.begin(), dec.end());
  for (size_t i = 0; i < dec.size();) {
    size_t j = i;
    while (j < dec.size() && dec[j].first == dec[i].first) j++;
    if ((int32_t)(j - i) > pool->rc[dec[i].first]) {
      zp::set_error("id %d released %zu times but its refcount is %d", dec[i].first, j - i,
                    pool->rc[dec[i].first]);
      return ZP_ERR_INVALID;
    }
    i = j;
  }
  int32_t k = 0;
  for (int32_t i = 0; i < n; i++) {
    if (--pool->rc[ids[i]] == 0) {
      pool->free_ids.insert(ids[i]);
      if (freed_out) freed_out[k] = ids[i];
      k++;
    }
  }
  if (n_freed) *n_freed = k;
  return ZP_OK;
}

int32_t zp_block_refcount(const zp_block_pool* pool, int32_t id) {
  if (!pool || id < 0 || id >= pool->num_blocks) return -1;
  return pool->rc[id];
}

int32_t zp_block_num_free(const zp_block_pool* pool) {
  if (!pool) return -1;
  const_cast<zp_block_pool*>(pool)->reap();
  return (int32_t)pool->free_ids.size();
}

int32_t zp_block_num_pending(const zp_block_pool* pool) {
  if (!pool) return -1;
  const_cast<zp_block_pool*>(pool)->reap();
  return pool->pending_count();
}

zp_status zp_block_pool_fence(zp_block_pool* pool) {
  zp::clear_error();
  if (!pool) { zp::set_error("pool is NULL"); return ZP_ERR_INVALID; }
  size_t keep = 0;
  for (size_t i = 0; i < pool->pending.size(); i++) {
    auto& p = pool->pending[i];
    if (p.event == nullptr) {
      for (int32_t id : p.ids) pool->free_ids.insert(id);
    } else {
      if (keep != i) pool->pending[keep] = std::move(p);
      keep++;
    }
  }
  pool->pending.resize(keep);
  return ZP_OK;
}

zp_status zp_block_pool_sync(zp_block_pool* pool) {
  zp::clear_error();
  if (!pool) { zp::set_error("pool is NULL"); return ZP_ERR_INVALID; }
  for (auto& p : pool->pending) {
    if (p.event) {
      hipError_t e = hipEventSynchronize(p.event);
      if (e != hipSuccess) {
        pool->poisoned = true;
        zp::set_error("hipEventSynchronize: %s", hipGetErrorString(e));
        return ZP_ERR_HIP;
      }
    }
  }
  for (auto& p : pool->pending) {
    for (int32_t id : p.ids) pool->free_ids.insert(id);
    pool->give_back_event(p.event);
  }
  pool->pending.clear();
  return ZP_OK;
}

zp_status zp_compress_plan(zp_block_pool* pool, int32_t n_max, int32_t num_reqs,
                           int32_t* block_tables, int32_t* src_out, int32_t* dst_out,
                           int32_t* freed_ids, int32_t* num_freed) {
  return zp_compress_plan_n(pool, n_max, n_max, num_reqs, block_tables, src_out, dst_out,
                            freed_ids, num_freed);
}

zp_status zp_compress_plan_n(zp_block_pool* pool, int32_t n_src, int32_t n_max, int32_t num_reqs,
                             int32_t* block_tables, int32_t* src_out, int32_t* dst_out,
                             int32_t* freed_ids, int32_t* num_freed) {
  zp::TraceRange trace("zp.compress_plan");
  zp::clear_error();
  if (num_reqs > 0 && (!src_out || !dst_out || !freed_ids || !num_freed)) {
    zp::set_error("output pointers must not be NULL");
    return ZP_ERR_INVALID;
  }
  zp::PlanResult plan;
  zp_status st = zp::plan_compression(pool, n_src, n_max, num_reqs, block_tables, &plan);
  if (st != ZP_OK) return st;
  if (num_reqs > 0) {
    std::memcpy(src_out, plan.src.data(), plan.src.size() * sizeof(int32_t));
    std::memcpy(dst_out, plan.dst.data(), plan.dst.size() * sizeof(int32_t));
    std::copy(plan.freed.begin(), plan.freed.end(), freed_ids);  // may be empty
  }
  if (num_freed) *num_freed = (int32_t)plan.freed.size();
  zp::add_pending(pool, std::move(plan.freed), nullptr);
  return ZP_OK;
}

}  // extern "C"
