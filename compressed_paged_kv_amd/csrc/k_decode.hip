// Paged decode attention, its split combine, and the KV append (gfx950).
//
// Decode reads each request's keys and values through its block table
// (upskillscore.com guide, "How it works": logical blocks map to arbitrary
// physical blocks).  It is a streaming, HBM-bound pass (4 flops per byte),
// so it runs on the vector ALUs: bf16 q.k through v_dot2c_f32_bf16 with
// float32 accumulation, p*v as float32 FMAs.
//
// Grid: x = split of the block list, y = KV head (and query-head subgroup),
// z = request.  A workgroup has 8 waves.  Within a wave, lane = LPT*t + c
// handles token t of a step of 64/LPT tokens and the c-th LPT-th of the head
// dimension, as 16-byte vectors at byte offsets 16*LPT*v + 16*c of the row,
// so one load instruction covers whole contiguous rows.  The steps of one
// block go to different waves (wave w takes step w % SPB of the blocks
// w / SPB, w / SPB + 8/SPB, ... counted from the newest), so all of a
// block's tile is requested at about the same time.  All G query heads of
// the KV head are done together, so K and V are read once for the group;
// blocks are walked newest first, and the next block's K and V are loaded
// before the current one is consumed.  V is loaded non-temporally: nothing
// reads it again soon, whereas K stays cached for the scoring of a
// compression that follows the decode step (measured: both faster).  The
// LPT lanes of a token add their partial dot products; every lane keeps its own
// running softmax state (max m, sum l, accumulator) for the tokens it saw,
// rescaled only when the max grows by more than 64 in log2 units (exact up
// to rounding: the final normalisation divides by the same stale max; terms
// stay below 2^64, far inside the float range), and the states of
// lanes, waves and splits are merged by log-sum-exp at the end.
#include <mutex>

#include "zp_device.h"
#include "zp_internal.h"

namespace zp {
namespace {

// Split partials of zp_paged_decode_noalloc, for callers that cannot
// allocate device memory.  Every GPU the library runs on holds its own copy
// until the process ends.  Host code never passes this name to a kernel (on
// the host it only stands for the variable): decode_static_scratch() looks
// up each device's address once and the kernels get that address.
static __device__ __align__(256) unsigned char scratch[kDecodeStaticScratchBytes];

constexpr float kInitMax = -1.0e30f;
constexpr float kLazy = 64.0f;
// Tuning knobs (defaults chosen by measurement on MI355X).
#ifndef ZP_DECODE_LANES_PER_TOKEN
#define ZP_DECODE_LANES_PER_TOKEN 16
#endif
#ifndef ZP_DECODE_PREFETCH
#define ZP_DECODE_PREFETCH 1  // steps loaded ahead of the one being consumed
#endif
constexpr int kLanesPerToken = ZP_DECODE_LANES_PER_TOKEN;  // lanes sharing one token row
constexpr int PD = ZP_DECODE_PREFETCH;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int DT>
struct Elem;

template <>
struct Elem<ZP_BF16> {
  static constexpr int kBytes = 2;
  // dot of 8 bf16 pairs (one 16-byte vector of q and k) added to acc
  __device__ static inline float dot(uint4 q, uint4 k, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, k.w), acc, false);
    return acc;
  }
  static constexpr int kPerVec = 8;
  __device__ static inline void unpack(uint4 v, float (&o)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      o[2 * k] = __uint_as_float(w[k] << 16);
      o[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
};

template <>
struct Elem<ZP_F32> {
  static constexpr int kBytes = 4;
  __device__ static inline float dot(uint4 q, uint4 k, float acc) {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
  static constexpr int kPerVec = 4;
  __device__ static inline void unpack(uint4 v, float (&o)[4]) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
};

__device__ inline uint4 ld16(const char* p) { return ldg16(p); }

// Sum over groups of LPT consecutive lanes (LPT = 4, 8 or 16) with DPP
// row permutations: xor 1 and xor 2 inside quads, then the half-row and
// row mirrors pair the 4- and 8-lane halves.  Every lane of the group ends
// with the same (commutatively added) value.
template <int LPT>
__device__ inline float group_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  if constexpr (LPT >= 8)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
  if constexpr (LPT >= 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
  return x;
}

// 2^x on the hardware unit (no denormal rescue: results below 2^-126 flush
// to zero, which only drops probabilities far below the output tolerance).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One output element, as float32 or (out_bf16) bfloat16 rounded to nearest
// even; NaN stays NaN.
__device__ inline void store_out(const DecodeParams& p, size_t idx, float x) {
  if (p.out_bf16) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t r = (x != x) ? 0x7FC0u : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    static_cast<uint16_t*>(p.out)[idx] = (uint16_t)r;
  } else {
    static_cast<float*>(p.out)[idx] = x;
  }
}

// Optional output: the log-sum-exp of the scaled logits of query head hq,
// ln sum_j exp(scale * q.k_j), from the merged (max M, sum L) in log2 units.
__device__ inline void store_lse(const DecodeParams& p, int r, int hq, float M, float L) {
  if (!p.lse) return;
  const int row = p.lse_rows ? p.lse_rows[r] : r;
  if (row < 0 || row >= p.lse_cap) return;
  p.lse[(size_t)row * p.Hq + hq] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -__builtin_inff();
}

// G here is the number of query heads one workgroup handles (at most 4, to
// keep the accumulators in registers); larger groups are split over
// blockIdx.y = kv_head * nsub + sub.
template <int DT, int D, int B, int G>
__global__ __launch_bounds__(kDecodeThreads) void k_decode(DecodeParams p) {
  constexpr int EB = Elem<DT>::kBytes;
  // lanes per token row: the knob, capped at one 16-byte vector per lane
  constexpr int LPT = (D * EB / 16 < kLanesPerToken) ? D * EB / 16 : kLanesPerToken;
  constexpr int TPS = 64 / LPT;                        // tokens per step
  constexpr int NV = D * EB / (16 * LPT);              // 16-byte vectors per lane per row
  constexpr int EPV = Elem<DT>::kPerVec;              // elements per vector
  constexpr int NE = NV * EPV;                         // = D / LPT
  constexpr int ROW = D * EB;
  constexpr int SPB = B / TPS;                         // steps per block
  constexpr int NW = kDecodeThreads / 64;              // waves per workgroup
  const int split = blockIdx.x, r = blockIdx.z;
  const int group = p.Hq / p.H, nsub = group / G;
  const int h = blockIdx.y / nsub, hq0 = h * group + (blockIdx.y - h * nsub) * G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok = lane / LPT, c = lane % LPT;

  // device-side lengths and ids are clamped / skipped so that a bad table
  // can never send a load outside the pools
  const int seq = min(max(p.seq_lens[r], 0), p.max_blocks * B);
  const int nblk = (seq + B - 1) / B;
  const int blk_begin = split * p.blocks_per_split;
  const int blk_end = min(blk_begin + p.blocks_per_split, nblk);

  uint4 q[G][NV];
#pragma unroll
  for (int g = 0; g < G; g++) {
    const char* qp = static_cast<const char*>(p.q) + ((size_t)r * p.Hq + hq0 + g) * ROW + c * 16;
#pragma unroll
    for (int v = 0; v < NV; v++) q[g][v] = ld16(qp + v * 16 * LPT);
  }
  // optional record of the query (split 0, wave 0, token lane group 0 hold
  // the whole row between them)
  if (p.q_rec && split == 0 && wave == 0 && tok == 0) {
    const int row = p.lse_rows ? p.lse_rows[r] : r;
    if (row >= 0 && row < p.lse_cap) {
#pragma unroll
      for (int g = 0; g < G; g++) {
        char* qo = static_cast<char*>(p.q_rec) + ((size_t)row * p.Hq + hq0 + g) * ROW + c * 16;
#pragma unroll
        for (int v = 0; v < NV; v++) stg16(qo + v * 16 * LPT, q[g][v]);
      }
    }
  }
  float m[G], l[G], acc[G][NE];
#pragma unroll
  for (int g = 0; g < G; g++) {
    m[g] = kInitMax;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; e++) acc[g][e] = 0.f;
  }

  const char* kb = static_cast<const char*>(p.k);
  const char* vb = static_cast<const char*>(p.v);
  const size_t tile_bytes = (size_t)B * ROW;
  // SPB waves share a block, one step each, so a block's tile is requested
  // at once; the workgroup walks NWB blocks at a time, newest first: this
  // wave's i-th block is blk_end - 1 - (wblk + NWB*i), always at step st.
  // The newest rows are the likeliest to be still in the memory-side cache
  // (appended tokens, and the tail of a compaction that has just rewritten
  // the request), and the oldest blocks, read last, are where a following
  // scoring pass starts.  The order changes nothing but rounding: every
  // lane's softmax state is merged by log-sum-exp at the end.
  static_assert(NW % SPB == 0, "steps per block must divide the waves");
  constexpr int NWB = NW / SPB;
  const int wblk = wave / SPB, st = wave - wblk * SPB;
  const int lane_off = (st * TPS + tok) * ROW + c * 16;  // this lane's bytes inside a block
  const int my_blocks = blk_end - blk_begin - wblk > 0 ? (blk_end - blk_begin - wblk + NWB - 1) / NWB : 0;
  // block of the wave's i-th item: wblk + NWB*i < blk_end - blk_begin for
  // every i < my_blocks, so it stays inside [blk_begin, blk_end)
  auto block_of = [&](int i) { return blk_end - 1 - (wblk + NWB * i); };
  for (int g0 = 0; g0 < my_blocks; g0 += 64) {
    const int nb_here = min(64, my_blocks - g0);
    int id = -1;
    if (lane < nb_here) {
      id = p.tables[(size_t)r * p.max_blocks + block_of(g0 + lane)];
      if ((unsigned)id >= (unsigned)p.num_blocks) id = -1;
    }
    const int n_items = nb_here;
    // item i = the wave's i-th block of the group.  Items past the end
    // re-read the last item and a skipped block reads row 0 of the pool:
    // the loads stay unconditional (straight-line code lets the compiler
    // count outstanding loads instead of draining them) and such items are
    // masked out below.
    auto item_base = [&](int item) -> long long {
      const int it = min(item, n_items - 1);
      const int pid = __builtin_amdgcn_readlane(id, it);
      if (pid < 0) return 0;
      return (long long)(((size_t)pid * p.H + h) * tile_bytes) + lane_off;
    };
    auto item_live = [&](int item) -> bool {
      if (item >= n_items) return false;
      const int pid = __builtin_amdgcn_readlane(id, item);
      return pid >= 0 && block_of(g0 + item) * B + st * TPS + tok < seq;
    };
    // ring of PD+1 register slots: item k lives in slot k % (PD+1) and is
    // loaded PD items before it is consumed
    uint4 kr[PD + 1][NV], vr[PD + 1][NV];
    auto fetch = [&](int item, uint4 (&kd)[NV], uint4 (&vd)[NV]) {
      const long long o = item_base(item);
#pragma unroll
      for (int v = 0; v < NV; v++) {
        kd[v] = ld16(kb + o + v * 16 * LPT);
        vd[v] = ldg16_stream(vb + o + v * 16 * LPT);
      }
    };
#pragma unroll
    for (int k = 0; k < PD; k++) fetch(k, kr[k], vr[k]);
    for (int base = 0; base < n_items; base += PD + 1) {
#pragma unroll
      for (int sl = 0; sl < PD + 1; sl++) {
        const int item = base + sl;
        fetch(item + PD, kr[(sl + PD) % (PD + 1)], vr[(sl + PD) % (PD + 1)]);
        // a skipped block, a token past the end or an item past the end
        // contributes nothing
        const bool live = item_live(item);
        // (its probability is forced to exactly 0 below: while a lane has
        // seen no live token its max is still kInitMax, and 2^(x - m) would
        // count a dead one as 1)
        float x[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
          float sdot = 0.f;
#pragma unroll
          for (int v = 0; v < NV; v++) sdot = Elem<DT>::dot(q[g][v], kr[sl][v], sdot);
          sdot = group_sum<LPT>(sdot);
          x[g] = live ? sdot * p.scale_log2 : kInitMax;
        }
        float vf[NE];
#pragma unroll
        for (int v = 0; v < NV; v++) {
          float tmp[EPV];
          Elem<DT>::unpack(vr[sl][v], tmp);
#pragma unroll
          for (int k = 0; k < EPV; k++) vf[v * EPV + k] = live ? tmp[k] : 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; g++) {
          if (x[g] > m[g] + kLazy) {
            const float cr = fast_exp2(m[g] - x[g]);
            l[g] *= cr;
#pragma unroll
            for (int e = 0; e < NE; e++) acc[g][e] *= cr;
            m[g] = x[g];
          }
          const float pr = live ? fast_exp2(x[g] - m[g]) : 0.f;
          l[g] += pr;
#pragma unroll
          for (int e = 0; e < NE; e++) acc[g][e] = fmaf(pr, vf[e], acc[g][e]);
        }
      }
    }
  }
  // merge the token lanes that share a head-dimension slice
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; g++) {
      const float m2 = __shfl_xor(m[g], off);
      const float l2 = __shfl_xor(l[g], off);
      const float M = fmaxf(m[g], m2);
      const float c1 = exp2f(m[g] - M), c2 = exp2f(m2 - M);
      l[g] = l[g] * c1 + l2 * c2;
#pragma unroll
      for (int e = 0; e < NE; e++) {
        const float a2 = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * c1 + a2 * c2;
      }
      m[g] = M;
    }
  }
  // merge the waves through LDS
  __shared__ float s_acc[NW][G][D];
  __shared__ float s_ml[NW][G][2];
  if (tok == 0) {
#pragma unroll
    for (int g = 0; g < G; g++) {
#pragma unroll
      for (int v = 0; v < NV; v++)
#pragma unroll
        for (int k = 0; k < EPV; k++)
          s_acc[wave][g][v * (16 * LPT / EB) + c * EPV + k] = acc[g][v * EPV + k];
      if (c == 0) {
        s_ml[wave][g][0] = m[g];
        s_ml[wave][g][1] = l[g];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int g = idx / D, d = idx - g * D;
    float M = s_ml[0][g][0];
#pragma unroll
    for (int w = 1; w < NW; w++) M = fmaxf(M, s_ml[w][g][0]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const float cw = exp2f(s_ml[w][g][0] - M);
      L = fmaf(s_ml[w][g][1], cw, L);
      o = fmaf(s_acc[w][g][d], cw, o);
    }
    const int hq = hq0 + g;
    if (p.nsplit == 1) {
      store_out(p, ((size_t)r * p.Hq + hq) * D + d, L > 0.f ? o / L : 0.f);
      if (d == 0) store_lse(p, r, hq, M, L);
    } else {
      float* part = p.partial + (((size_t)r * p.Hq + hq) * p.nsplit + split) * (D + 2);
      part[2 + d] = o;
      if (d == 0) {
        part[0] = M;
        part[1] = L;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void k_decode_combine(DecodeParams p) {
  const int rh = blockIdx.x;  // r * Hq + hq
  const int d = threadIdx.x;
  const float* part = p.partial + (size_t)rh * p.nsplit * (D + 2);
  float M = kInitMax;
  for (int s = 0; s < p.nsplit; s++) M = fmaxf(M, part[(size_t)s * (D + 2)]);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < p.nsplit; s++) {
    const float* ps = part + (size_t)s * (D + 2);
    const float c = exp2f(ps[0] - M);
    L = fmaf(ps[1], c, L);
    o = fmaf(ps[2 + d], c, o);
  }
  store_out(p, (size_t)rh * D + d, L > 0.f ? o / L : 0.f);
  if (d == 0) store_lse(p, rh / p.Hq, rh % p.Hq, M, L);
}

__global__ __launch_bounds__(256) void k_append(AppendParams p) {
  const int r = blockIdx.x;
  const int slot = p.slot_mapping[r];
  if (slot < 0) return;
  const int blk = slot / p.block_size, off = slot - blk * p.block_size;
  if (blk >= p.num_blocks) return;
  const int vpr = p.row_bytes / 16;
  const int per_pool = p.H * vpr;
  for (int idx = threadIdx.x; idx < 2 * per_pool; idx += blockDim.x) {
    const int kv = idx / per_pool, rem = idx - kv * per_pool;
    const int h = rem / vpr, vec = rem - h * vpr;
    const char* from = static_cast<const char*>(kv ? p.v_new : p.k_new) +
                       ((size_t)r * p.H + h) * p.row_bytes + vec * 16;
    char* to = static_cast<char*>(kv ? p.v : p.k) +
               (((size_t)blk * p.H + h) * p.block_size + off) * p.row_bytes + vec * 16;
    stg16(to, ldg16(from));
  }
}

template <int DT, int D, int B>
hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
  const int group = p.Hq / p.H;
  const int per_wg = group < 4 ? group : 4;
  dim3 grid(p.nsplit, p.H * (group / per_wg), p.R), block(kDecodeThreads);
  if (per_wg != 1 && per_wg != 2 && per_wg != 4) return hipErrorInvalidValue;
  prof_begin(ZP_PHASE_DECODE, s);
  switch (per_wg) {
    case 1: hipLaunchKernelGGL((k_decode<DT, D, B, 1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_decode<DT, D, B, 2>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_decode<DT, D, B, 4>), grid, block, 0, s, p); break;
  }
  prof_end(ZP_PHASE_DECODE, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  prof_begin(ZP_PHASE_COMBINE, s);
  hipLaunchKernelGGL((k_decode_combine<D>), dim3(p.R * p.Hq), dim3(D), 0, s, p);
  prof_end(ZP_PHASE_COMBINE, s);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_d(const DecodeParams& p, int block_size, hipStream_t s) {
  if (block_size == 16) return launch_g<DT, D, 16>(p, s);
  if (block_size == 32) return launch_g<DT, D, 32>(p, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const DecodeParams& p, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 64) return launch_d<DT, 64>(p, block_size, s);
  if (head_dim == 128) return launch_d<DT, 128>(p, block_size, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int block_size,
                         hipStream_t s) {
  if (p.R <= 0) return hipSuccess;
  if (dtype == ZP_BF16) return launch_dt<ZP_BF16>(p, head_dim, block_size, s);
  if (dtype == ZP_F32) return launch_dt<ZP_F32>(p, head_dim, block_size, s);
  return hipErrorInvalidValue;
}

hipError_t decode_static_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  if (p.R <= 0) return hipSuccess;
  prof_begin(ZP_PHASE_APPEND, s);
  hipLaunchKernelGGL(k_append, dim3(p.R), dim3(256), 0, s, p);
  prof_end(ZP_PHASE_APPEND, s);
  return hipGetLastError();
}

}  // namespace zp
