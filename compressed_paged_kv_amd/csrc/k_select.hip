// Per-head survivor selection of the compression pass (gfx950).
//
// For every (layer, request, KV head) the candidates are slots j < C = T - w
// with score s[j]; the window slots C..T-1 always survive (ko page section
// 2.A).  K_sel candidates survive, so exactly E = C - K_sel are evicted: the
// E smallest under the order (s ascending, then slot descending), i.e. on
// equal scores the higher slot goes first and the lower one is kept.
//
// One workgroup (256 threads) per unit; thread t owns the contiguous slots
// [t*PER, (t+1)*PER).  Scores become order-preserving 32-bit keys (-0 folded
// into +0).  A radix select over the keys (4 passes of 8 bits, LDS histogram
// and block scan) finds the E-th smallest key tau and how many keys equal to
// tau must go; block-wide prefix counts in slot order then give which tied
// slots are the highest, and where each evicted slot lands in the ascending
// output list.  Optionally the full ascending survivor list is written too.
#include "zp_internal.h"

namespace zp {
namespace {

constexpr int kThreads = 256;

__device__ inline uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);  // -0 + 0 = +0 under round-to-nearest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive block-wide sum; `scratch` holds >= 4 ints.  Ends with a barrier
// so scratch may be reused afterwards.
__device__ inline int block_incl_sum(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; w++) before += scratch[w];
  __syncthreads();
  return v + before;
}

__device__ inline int block_total(int incl_last_thread, int* scratch) {
  // broadcast the inclusive sum of the last thread
  if (threadIdx.x == kThreads - 1) scratch[4] = incl_last_thread;
  __syncthreads();
  const int t = scratch[4];
  __syncthreads();
  return t;
}

template <int PER>
__global__ __launch_bounds__(kThreads) void k_select(SelectParams p) {
  const size_t unit = blockIdx.x;
  const int tid = threadIdx.x;
  const float* s = p.score + unit * p.T;
  __shared__ int hist[256];
  __shared__ int scratch[8];
  __shared__ int sel[2];

  uint32_t key[PER];
#pragma unroll
  for (int k = 0; k < PER; k++) {
    const int j = tid * PER + k;
    key[k] = (j < p.C) ? order_key(s[j]) : 0xFFFFFFFFu;
  }

  // radix select of the E-th smallest candidate key (rank counted from 1)
  uint32_t prefix = 0, pmask = 0;
  int rank = p.E;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int j = tid * PER + k;
      if (j < p.C && (key[k] & pmask) == prefix) atomicAdd(&hist[(key[k] >> shift) & 0xFFu], 1);
    }
    __syncthreads();
    const int cnt = hist[tid];
    const int incl = block_incl_sum(cnt, scratch);
    if (incl - cnt < rank && incl >= rank) {
      sel[0] = tid;
      sel[1] = incl - cnt;
    }
    __syncthreads();
    prefix |= (uint32_t)sel[0] << shift;
    pmask |= 0xFFu << shift;
    rank -= sel[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;
  const int evict_ties = rank;  // how many candidates with key == tau are evicted

  // ties: the evict_ties highest slots among key == tau go
  int my_ties = 0;
#pragma unroll
  for (int k = 0; k < PER; k++) my_ties += (tid * PER + k < p.C && key[k] == tau) ? 1 : 0;
  const int ties_incl = block_incl_sum(my_ties, scratch);
  const int ties_total = block_total(ties_incl, scratch);
  int tie_rank = ties_incl - my_ties;  // ties at lower slots
  bool ev[PER];
  int my_ev = 0;
#pragma unroll
  for (int k = 0; k < PER; k++) {
    const int j = tid * PER + k;
    bool e = false;
    if (j < p.C) {
      if (key[k] < tau) {
        e = true;
      } else if (key[k] == tau) {
        e = tie_rank >= ties_total - evict_ties;
        tie_rank++;
      }
    }
    ev[k] = e;
    my_ev += e ? 1 : 0;
  }
  const int ev_incl = block_incl_sum(my_ev, scratch);
  int pos = ev_incl - my_ev;
  int32_t* out = p.evicted + unit * p.E;
#pragma unroll
  for (int k = 0; k < PER; k++)
    if (ev[k] && pos < p.E) out[pos++] = tid * PER + k;

  if (p.dbg_kept) {
    int my_keep = 0;
#pragma unroll
    for (int k = 0; k < PER; k++) my_keep += (tid * PER + k < p.T && !ev[k]) ? 1 : 0;
    const int keep_incl = block_incl_sum(my_keep, scratch);
    int kp = keep_incl - my_keep;
    int32_t* kout = p.dbg_kept + unit * p.K_keep;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int j = tid * PER + k;
      if (j < p.T && !ev[k] && kp < p.K_keep) kout[kp++] = j;
    }
  }
}

}  // namespace

int select_per_thread(int T) {
  const int need = (T + kThreads - 1) / kThreads;
  int per = 1;
  while (per < need) per <<= 1;
  return per <= 32 ? per : 0;
}

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
  if (p.units <= 0) return hipSuccess;
  dim3 grid(p.units), block(kThreads);
  const int per = select_per_thread(p.T);
  if (per == 0) return hipErrorInvalidValue;
  prof_begin(ZP_PHASE_SELECT, s);
  switch (per) {
    case 1: hipLaunchKernelGGL(k_select<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(k_select<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(k_select<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(k_select<8>, grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL(k_select<16>, grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL(k_select<32>, grid, block, 0, s, p); break;
  }
  prof_end(ZP_PHASE_SELECT, s);
  return hipGetLastError();
}

}  // namespace zp
