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
// same physical row (unmoved prefix of an in-place block) are not written,
// and the walk starts at the first row that moves: before the first evicted
// slot and the first re-targeted block nothing changes.
//
// Grid: x = (head, K|V), y = (layer, request).  256 threads; each row of
// d * elem_bytes bytes is VPR 16-byte vectors, one per thread, U rows per
// thread per tile.
#include "zp_device.h"
#include "zp_internal.h"

namespace zp {
namespace {

constexpr int kThreads = 256;
#ifndef ZP_COMPACT_UNROLL
#define ZP_COMPACT_UNROLL 6  // rows per thread per tile
#endif
constexpr int kUnroll = ZP_COMPACT_UNROLL;
constexpr int kMaxSlots = 8192;    // K_keep bound (T = n_src * block_size <= 8192, checked on the host)
constexpr int kMaxBlocks = 512;    // n_src bound for the LDS block tables (T <= 8192, b >= 16)
#ifndef ZP_COMPACT_STREAM
#define ZP_COMPACT_STREAM 2  // 1: non-temporal stores, 2: non-temporal loads and stores
#endif

template <int VPR, int B>
__global__ __launch_bounds__(kThreads, 4) void k_compact(CompactParams p) {
  constexpr int kRowsPerPass = kThreads / VPR;
  constexpr int kRowsPerTile = kRowsPerPass * kUnroll;
  const int h = blockIdx.x >> 1, kv = blockIdx.x & 1;
  const int lr = p.layer0 * p.R + blockIdx.y;   // (layer, request) over the whole call
  const int l = lr / p.R, r = lr - l * p.R;
  const int tid = threadIdx.x;
  const int vec = tid % VPR, rsub = tid / VPR;
  const size_t unit = (size_t)lr * p.H + h;
  constexpr int b = B;
  constexpr size_t row_bytes = (size_t)VPR * 16;

  __shared__ int f[kMaxEvicted];
  __shared__ int srcb[kMaxBlocks];
  __shared__ int dstb[kMaxBlocks];
  __shared__ unsigned short kept[kMaxSlots];
  __shared__ int s_first;
  // this request's blocks (the call's largest unless rows are ragged) and evictions
  const int n_src = unit_blocks(p.src, p.src_stride, r, p.n_src, p.n_max, p.ragged);
  const int E = n_src * b - p.K_keep;
  const int32_t* ev = p.evicted + unit * p.E;  // stride: the call's largest E
  for (int i = tid; i < E; i += kThreads) f[i] = ev[i] - i;
  // an id outside the pool is read as block 0 and never written
  for (int n = tid; n < n_src; n += kThreads) {
    const int id = p.src[(size_t)r * p.src_stride + n];
    srcb[n] = (unsigned)id < (unsigned)p.num_blocks ? id : 0;
  }
  for (int n = tid; n < p.n_max - 1; n += kThreads) {
    const int id = p.dst[(size_t)r * p.dst_stride + n];
    dstb[n] = (unsigned)id < (unsigned)p.num_blocks ? id : -1;
  }
  if (tid == 0) s_first = E > 0 ? ev[0] : p.K_keep;  // rows below the first eviction stay put
  __syncthreads();
  // ... unless their block is re-targeted (a new block for a shared source)
  for (int n = tid; n < p.n_max - 1; n += kThreads)
    if (dstb[n] != srcb[n]) atomicMin(&s_first, n * b);
  __syncthreads();
  const int first = min(s_first, p.K_keep);
  // survivor list, once per workgroup: kept[r] = r + #{i : f_i <= r}
  for (int row = tid; row < p.K_keep; row += kThreads) {
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (f[mid] <= row) lo = mid + 1; else hi = mid;
    }
    kept[row] = (unsigned short)(row + lo);
  }
  __syncthreads();

  // a row of the pool as one index (block, head, offset), below 2^31 for
  // any pool the host accepts; the byte address is formed at the access
  const LayerArgs& la = p.layers[l - p.layer0];
  char* const base = static_cast<char*>(kv ? la.v : la.k) + vec * 16;
  auto row_of = [&](int blk, int off) -> int { return (blk * p.H + h) * b + off; };
  auto addr = [&](int row) -> char* { return base + (size_t)(unsigned)row * row_bytes; };
  // Rows past the end are clamped to the last row; an unmoved row is read
  // but not written (target -1).  Loads stay unconditional, so the compiler
  // can keep the next tile's loads in flight while this tile is stored.
  auto load_tile = [&](int t0, uint4 (&buf)[kUnroll], int (&to)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int row = min(t0 + rsub + u * kRowsPerPass, p.K_keep - 1);
      const int j = kept[row];
      const int from = row_of(srcb[j / b], j % b);
      const int db = dstb[row / b];
      const int dst = row_of(db, row % b);
      buf[u] = ZP_COMPACT_STREAM >= 2 ? ldg16_stream(addr(from)) : ldg16(addr(from));
      to[u] = (db >= 0 && dst != from && t0 + rsub + u * kRowsPerPass < p.K_keep) ? dst : -1;
    }
  };
  if (first >= p.K_keep) return;  // nothing moves (uniform across the workgroup)
  uint4 cur[kUnroll], nxt[kUnroll];
  int cur_to[kUnroll];
  int nxt_to[kUnroll];
  load_tile(first, cur, cur_to);
  for (int t0 = first; t0 < p.K_keep; t0 += kRowsPerTile) {
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
      if (cur_to[u] >= 0) {
        if (ZP_COMPACT_STREAM >= 1) stg16_stream(addr(cur_to[u]), cur[u]); else stg16(addr(cur_to[u]), cur[u]);
      }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      cur[u] = nxt[u];
      cur_to[u] = nxt_to[u];
    }
  }
}

}  // namespace

template <int VPR>
void launch_vpr(const CompactParams& p, dim3 grid, int block_size, hipStream_t s) {
  if (block_size == 16)
    hipLaunchKernelGGL((k_compact<VPR, 16>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_compact<VPR, 32>), grid, dim3(kThreads), 0, s, p);
}

hipError_t launch_compact(const CompactParams& p, int num_layers, int row_bytes, int block_size,
                          hipStream_t s) {
  if (p.R <= 0) return hipSuccess;
  if (p.E > kMaxEvicted || p.n_src > kMaxBlocks || p.n_max > p.n_src || p.K_keep > kMaxSlots)
    return hipErrorInvalidValue;
  if (block_size != 16 && block_size != 32) return hipErrorInvalidValue;
  if (p.K_keep != (p.n_max - 1) * block_size) return hipErrorInvalidValue;
  if (num_layers < 1 || num_layers > kArgLayers) return hipErrorInvalidValue;
  dim3 grid(2 * p.H, num_layers * p.R);   // layers layer0 .. layer0 + num_layers - 1
  const int vpr = row_bytes / 16;
  if (vpr != 8 && vpr != 16 && vpr != 32) return hipErrorInvalidValue;
  prof_begin(ZP_PHASE_COMPACT, s);
  switch (vpr) {
    case 8: launch_vpr<8>(p, grid, block_size, s); break;
    case 16: launch_vpr<16>(p, grid, block_size, s); break;
    case 32: launch_vpr<32>(p, grid, block_size, s); break;
  }
  prof_end(ZP_PHASE_COMPACT, s);
  return hipGetLastError();
}

}  // namespace zp
