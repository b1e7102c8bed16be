// Host-side block pool: reference counts, smallest-id-first free set, and
// groups of freed blocks that wait for the GPU work still reading them.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <set>
#include <vector>

#include "zp.h"

struct zp_block_pool {
  struct Pending {
    hipEvent_t event = nullptr;  // null: released by zp_block_pool_fence/sync
    std::vector<int32_t> ids;
  };
  int32_t num_blocks = 0;
  uint32_t flags = 0;
  bool poisoned = false;
  std::vector<int32_t> rc;
  std::set<int32_t> free_ids;
  std::vector<Pending> pending;
  // Events of completed groups, kept for the next group instead of being
  // destroyed and created again (event creation is a driver call per
  // compression otherwise).
  std::vector<hipEvent_t> spare_events;

  bool manual_fence() const { return (flags & ZP_POOL_MANUAL_FENCE) != 0; }
  // Move every pending group whose GPU work is done into the free set.
  void reap();
  // An event for a new pending group (a spare one, else a new one).
  hipError_t take_event(hipEvent_t* out);
  void give_back_event(hipEvent_t e);
  int32_t pending_count() const;
};

namespace zp {

// Output of the planner for one compression call.
struct PlanResult {
  std::vector<int32_t> src;    // [R][n_src]
  std::vector<int32_t> dst;    // [R][n_max-1]
  std::vector<int32_t> freed;  // ids whose refcount reached 0
};

// Validate and plan one compression call of requests holding n_src >= n_max
// blocks (tables [R][n_src]); on success updates the pool and the tables
// (n_max new ids, then -1 for the released surplus) and returns the plan
// (freed ids are NOT yet pending: the caller attaches them with
// add_pending).  On failure nothing changes.
//
// first_evict (optional, [R]): request r's lowest evicted slot over all its
// layers and heads.  A shared block n < n_max-1 with (n+1)*b <= first_evict[r]
// keeps its place and contents in every layer and head, so it stays in the
// table, shared, instead of being re-targeted.  With dry_run, only the
// checks of the tables run (not the free-block count; nothing changes).
//
// num_blocks (optional, [R]): request r holds only the first num_blocks[r]
// entries of its row (n_max <= num_blocks[r] <= n_src); the rest of the row
// must be -1 and is left so.
zp_status plan_compression(zp_block_pool* pool, int32_t n_src, int32_t n_max, int32_t num_reqs,
                           int32_t* block_tables, PlanResult* out,
                           const int32_t* first_evict = nullptr, int32_t block_size = 0,
                           bool dry_run = false, const int32_t* num_blocks = nullptr);

// Attach freed ids to a pending group released by `event` (or by a fence
// when event is null).  Takes ownership of the event.
void add_pending(zp_block_pool* pool, std::vector<int32_t> ids, hipEvent_t event);

}  // namespace zp
