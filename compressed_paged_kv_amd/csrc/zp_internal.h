// Internal declarations of the HIP library: launch parameters, launchers and
// error helpers.  Not part of the public ABI (that is include/zp.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "zp.h"

namespace zp {

// Thread-local error message behind zp_last_error().
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per-layer device pointers of the compression kernels, passed in the
// kernel arguments (no upload): K pool, V pool, window queries and the
// recorded window normalisers (or null).  One launch covers at most
// kArgLayers layers; more layers take several launches.
struct LayerArgs {
  void* k;
  void* v;
  const void* q;
  const float* lse;
};
constexpr int kArgLayers = 48;

// Largest number of (query head, window row) pairs per KV head, and the
// largest cached length the in-LDS scoring and selection handle.
constexpr int kMaxScoreRows = 128;
constexpr int kMaxScoreSlots = 8192;
// Largest eviction count per (layer, request, head) the compaction's LDS list
// holds: E = block_size * (n_src - n_max + 1).
constexpr int kMaxEvicted = 1024;
// Largest block count of one request in a compression call (n_src).
constexpr int kMaxCompressBlocks = 512;
// Largest T of the all-pairs redundancy (inverse norms of all keys in LDS).
constexpr int kMaxRedundancySlots = 8192;
// Paged decode: threads per workgroup, and the workgroup count below which
// a request's block list is split over several workgroups.
#ifndef ZP_DECODE_THREADS
#define ZP_DECODE_THREADS 512
#endif
constexpr int kDecodeThreads = ZP_DECODE_THREADS;
#ifndef ZP_DECODE_TARGET_WORKGROUPS
#define ZP_DECODE_TARGET_WORKGROUPS 512
#endif
constexpr int kDecodeTargetWorkgroups = ZP_DECODE_TARGET_WORKGROUPS;
// Fixed device scratch of the allocation-free decode entry point: the split
// partials [R][Hq][nsplit][d + 2] floats.  A list is split only while the
// (request, KV head, query subgroup) units number fewer than
// kDecodeTargetWorkgroups, so R*Hq*nsplit < 2 * 4 * kDecodeTargetWorkgroups
// (at most 4 query heads per unit) and the partials never exceed the bound
// below at head_dim 128.
constexpr size_t kDecodeStaticScratchBytes = size_t(4) << 20;
static_assert((size_t)2 * 4 * kDecodeTargetWorkgroups * (128 + 2) * sizeof(float) <=
                  kDecodeStaticScratchBytes,
              "the static decode scratch must hold the largest split partials");

struct ScoreParams {
  LayerArgs layers[kArgLayers];  // layers layer0 .. layer0 + launched layers - 1
  int32_t layer0;           // first layer of this launch; unit = layer0*R*H + blockIdx.x
  const int32_t* src;       // device, row r at src + r*src_stride: the request's n_src >= n_max blocks
  int32_t src_stride;
  int32_t dst_stride;       // row stride of dst
  int32_t* evicted;         // [L*R*H][E], ascending
  float* dbg_importance;    // optional [L*R*H][T]
  float* dbg_redundancy;    // optional [L*R*H][T]
  float* dbg_score;         // optional [L*R*H][T]
  int32_t* dbg_kept;        // optional [L*R*H][K_keep]
  int64_t* dbg_times;       // optional [L*R*H][5]: wall clock at the phase boundaries
  const int32_t* dst;       // device, row r at dst + r*dst_stride: the n_max-1 target blocks; compact in the same kernel; null: select only
  int32_t k_cached;         // fused compaction: load K normally (1) or non-temporally (0)
  // ragged: request r holds the blocks of its source row up to its first -1
  // (at least n_max); n_src, T, C and E are then the call's largest, and the
  // strides of evicted and of the debug arrays
  int32_t ragged;
  int32_t num_blocks;       // pool size: ids outside [0, num_blocks) are never followed
  // window rows from a query-slot store: request r's window position i is row
  // qslot[r]*w + i of the layer's q (and lse) arrays, a slot outside
  // [0, qslots) read as slot 0; null: row r*w + i
  const int32_t* qslot;
  int32_t qslots;
  int32_t R, H, Hq, G, w, n_src, n_max, T, C, E, K_keep, rows;  // T = n_src * b
  float scale_log2;  // log2(e) / sqrt(d)
};

struct CompactParams {
  LayerArgs layers[kArgLayers];  // layers layer0 .. layer0 + launched layers - 1
  int32_t layer0;
  const int32_t* src;       // device, row r at src + r*src_stride (n_src entries)
  const int32_t* dst;       // device, row r at dst + r*dst_stride (n_max-1 entries)
  int32_t src_stride, dst_stride;
  const int32_t* evicted;   // [L*R*H][E]
  int32_t ragged;           // as ScoreParams::ragged (E = the stride of evicted)
  int32_t num_blocks;
  int32_t R, H, n_src, n_max, E, K_keep;
};


struct DecodeParams {
  const void* k;
  const void* v;
  const void* q;            // [R][Hq][d]
  const int32_t* tables;    // [R][max_blocks]
  const int32_t* seq_lens;  // [R]
  void* out;                // [R][Hq][d], float32, or bfloat16 when out_bf16
  int32_t out_bf16;
  float* partial;           // [R][Hq][nsplit][d + 2]
  float* lse;               // optional [lse_cap][Hq]: natural-log normaliser per query head
  void* q_rec;              // optional [lse_cap][Hq][d]: copy of the query (cache dtype)
  const int32_t* lse_rows;  // optional [R]: row of lse / q_rec for request r (default r; < 0 skips)
  int32_t R, H, Hq, max_blocks, nsplit, blocks_per_split, num_blocks, lse_cap;
  float scale_log2;
};

struct RedundancyParams {
  const void* k;            // K pool of the layer
  const int32_t* tables;    // [R][n_blocks]
  float* out;               // [R][H][n_blocks * b]
  int32_t R, H, n_blocks, num_blocks;
};

struct AppendParams {
  void* k;
  void* v;
  const void* k_new;  // [R][H][d]
  const void* v_new;
  const int32_t* slot_mapping;
  int32_t R, H, block_size, row_bytes, num_blocks;
};

// Launchers (defined in the .hip files); they only check the template
// dispatch and enqueue.  Return hipSuccess or the launch error.
hipError_t launch_score(const ScoreParams& p, int dtype, int head_dim, int block_size, int units,
                        hipStream_t s);
// Workgroups of the scoring kernel (fused with the compaction, or selecting
// only) that one compute unit of the current device holds at once.
hipError_t score_resident_per_cu(int dtype, int head_dim, int block_size, int rows, int T,
                                 bool fused, int* per_cu);
hipError_t launch_compact(const CompactParams& p, int num_layers, int row_bytes, int block_size,
                          hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int block_size,
                         hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
// Device address of the current device's copy of the fixed decode scratch
// (kDecodeStaticScratchBytes, 256-byte aligned), looked up once per device.
hipError_t decode_static_scratch(void** ptr);
hipError_t launch_redundancy_all(const RedundancyParams& p, int dtype, int head_dim,
                                 int block_size, hipStream_t s);
// Copies bytes (a multiple of 16, 16-byte aligned ends) from device-visible
// pinned host memory to device memory with a kernel on stream s.
hipError_t launch_upload(const void* host_src, void* dst, size_t bytes, hipStream_t s);
// host_out[r] = min over layers l and heads h of evicted[((l*R + r)*H + h)*E]
// (host_out: device address of host-mapped memory).
hipError_t launch_first_evict(const int32_t* evicted, int32_t* host_out, int R, int H, int L, int E,
                              hipStream_t s);

// Debug switches (ZP_DEBUG_* of zp.h), read from the environment on first
// use; roctx ranges on the host timeline while ZP_DEBUG_TRACE is set (a
// no-op otherwise, or when no roctx library can be loaded).
uint32_t debug_flags();
bool trace_available();
class TraceRange {
 public:
  explicit TraceRange(const char* name);
  ~TraceRange();
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;

 private:
  bool active_ = false;
};

// Kernel timing (no-ops unless enabled by zp_profile_enable): bracket one
// phase on stream s.
void prof_begin(int phase, hipStream_t s);
void prof_end(int phase, hipStream_t s);

// Geometry of the scoring kernel, shared by the host validation and the
// launcher.  Window rows come in 1, 2, 4 or 8 tiles of 16 (0: too many).
inline int score_row_tiles(int rows) {
  if (rows <= 0 || rows > kMaxScoreRows) return 0;
  const int t = (rows + 15) / 16;
  int p2 = 1;
  while (p2 < t) p2 <<= 1;
  return p2;
}
// More than 64 rows take two row groups, which keep three T-long arrays in
// LDS (T <= 4096, which also keeps a wave's block count within one id per
// lane).  At 64 rows or fewer one group is faster: with two, each block is
// read by two waves and the second read often misses L2.
inline bool score_two_groups(int row_tiles, int T) { return row_tiles > 4 && T <= 4096; }
// The fused scoring + selection kernel handles this shape.
inline bool score_fits(int rows, int T) {
  const int rt = score_row_tiles(rows);
  if (rt == 0 || T > kMaxScoreSlots) return false;
  return rt <= 4 || score_two_groups(rt, T);
}

}  // namespace zp
