// Order-preserving compaction of the compression pass (gfx950).
//
// For every (layer, request, KV head) and for K and V separately, logical
// slot r < K_keep of the target blocks receives old logical slot kept[r]
// (nl page Methodologie item 1: survivors move into the first N_max-1
// blocks; ko page section 2.C: shared blocks are never written, their
// survivors go to new target blocks).  The survivor list is rebuilt in LDS
// from the ascending evicted slots e_0 < e_1 < ...: with f_i = e_i - i,
//   kept[r] = r + #{ i : f_i <= r }   (one binary search per row).
//
// In-place safety.  A target block is either a fresh block (no one reads it)
// or the source block of the same logical position (private block).  Then
// writing slot r can only clobber old slot r, which is read by the row r'
// with kept[r'] = r, and r' <= r.  One workgroup walks the rows in ascending
// tiles; inside a tile every load has returned before the barrier and
// every store comes after it, so no store of a tile reaches a slot that
// the tile (or an earlier one) still has to read, and later tiles only read
// slots >= their first row -- which is also why the next tile's loads may be
// issued before this tile's stores.  Rows whose source and target are the
// same physical row (unmoved prefix of an in-place block) are not written.
//
// Grid: x = (head, K|V), y = (layer, request).  256 threads; each row of
// d * elem_bytes bytes is VPR 16-byte vectors, one per thread, U rows per
// thread per tile.
#include "zp_device.h"
#include "zp_internal.h"

namespace zp {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kMaxEvicted = 1024;  // E = block_size * (blocks beyond N_max - 1)
constexpr int kMaxSlots = 8192;    // T = n_max * block_size (the host checks the same)
constexpr int kMaxBlocks = 512;    // n_max bound for the LDS block tables (T <= 8192, b >= 16)
#ifndef ZP_COMPACT_STREAM
#define ZP_COMPACT_STREAM 2  // 1: non-temporal stores, 2: non-temporal loads and stores
#endif

template <int VPR>
__global__ __launch_bounds__(kThreads) void k_compact(CompactParams p) {
  constexpr int kRowsPerPass = kThreads / VPR;
  constexpr int kRowsPerTile = kRowsPerPass * kUnroll;
  const int h = blockIdx.x >> 1, kv = blockIdx.x & 1;
  const int lr = blockIdx.y;
  const int l = lr / p.R, r = lr - l * p.R;
  const int tid = threadIdx.x;
  const int vec = tid % VPR, rsub = tid / VPR;
  const size_t unit = (size_t)lr * p.H + h;
  const int b = p.K_keep / (p.n_max - 1);
  const size_t row_bytes = (size_t)VPR * 16;

  __shared__ int f[kMaxEvicted];
  __shared__ int srcb[kMaxBlocks];
  __shared__ int dstb[kMaxBlocks];
  __shared__ unsigned short kept[kMaxSlots];
  const int32_t* ev = p.evicted + unit * p.E;
  for (int i = tid; i < p.E; i += kThreads) f[i] = ev[i] - i;
  for (int n = tid; n < p.n_max; n += kThreads) srcb[n] = p.src[(size_t)r * p.n_max + n];
  for (int n = tid; n < p.n_max - 1; n += kThreads) dstb[n] = p.dst[(size_t)r * (p.n_max - 1) + n];
  __syncthreads();
  // survivor list, once per workgroup: kept[r] = r + #{i : f_i <= r}
  for (int row = tid; row < p.K_keep; row += kThreads) {
    int lo = 0, hi = p.E;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (f[mid] <= row) lo = mid + 1; else hi = mid;
    }
    kept[row] = (unsigned short)(row + lo);
  }
  __syncthreads();

  char* base = static_cast<char*>(p.layer_ptrs[l * kPtrsPerLayer + kv]);
  const size_t head_stride = (size_t)b * row_bytes;          // one (block, head) tile
  const size_t block_stride = (size_t)p.H * head_stride;    // one physical block
  auto row_addr = [&](int blk, int off) -> char* {
    return base + (size_t)blk * block_stride + h * head_stride + (size_t)off * row_bytes + vec * 16;
  };
  // Rows past the end are clamped to the last row; an unmoved row is read
  // but not written.  Loads stay unconditional, so the compiler can keep
  // the next tile's loads in flight while this tile is stored.
  auto load_tile = [&](int t0, uint4 (&buf)[kUnroll], char* (&to)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int row = min(t0 + rsub + u * kRowsPerPass, p.K_keep - 1);
      const int j = kept[row];
      const char* from = row_addr(srcb[j / b], j % b);
      char* dst = row_addr(dstb[row / b], row % b);
      buf[u] = ZP_COMPACT_STREAM >= 2 ? ldg16_stream(from) : ldg16(from);
      to[u] = (dst != from && t0 + rsub + u * kRowsPerPass < p.K_keep) ? dst : nullptr;
    }
  };
  uint4 cur[kUnroll], nxt[kUnroll];
  char* cur_to[kUnroll];
  char* nxt_to[kUnroll];
  load_tile(0, cur, cur_to);
  for (int t0 = 0; t0 < p.K_keep; t0 += kRowsPerTile) {
    load_tile(min(t0 + kRowsPerTile, p.K_keep - 1), nxt, nxt_to);
    // Every load of this tile must have returned its data before any thread
    // of the tile stores: the empty asm consumes the loaded registers, so the
    // compiler waits for them (and only them) ahead of the barrier.
#pragma unroll
    for (int u = 0; u < kUnroll; u++)
      asm volatile("" ::"v"(cur[u].x), "v"(cur[u].y), "v"(cur[u].z), "v"(cur[u].w));
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnroll; u++)
      if (cur_to[u]) {
        if (ZP_COMPACT_STREAM >= 1) stg16_stream(cur_to[u], cur[u]); else stg16(cur_to[u], cur[u]);
      }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      cur[u] = nxt[u];
      cur_to[u] = nxt_to[u];
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactParams& p, int num_layers, int row_bytes, int block_size,
                          hipStream_t s) {
  (void)block_size;
  if (p.R <= 0) return hipSuccess;
  if (p.E > kMaxEvicted || p.n_max > kMaxBlocks || p.K_keep > kMaxSlots) return hipErrorInvalidValue;
  dim3 grid(2 * p.H, num_layers * p.R), block(kThreads);
  const int vpr = row_bytes / 16;
  if (vpr != 8 && vpr != 16 && vpr != 32) return hipErrorInvalidValue;
  prof_begin(ZP_PHASE_COMPACT, s);
  switch (vpr) {
    case 8: hipLaunchKernelGGL(k_compact<8>, grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL(k_compact<16>, grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL(k_compact<32>, grid, block, 0, s, p); break;
  }
  prof_end(ZP_PHASE_COMPACT, s);
  return hipGetLastError();
}

}  // namespace zp
