// All-pairs redundancy of the keys of one layer (gfx950): for every
// (request, KV head) and each of its T = n_blocks*b slots j,
//   R_all[j] = 1/(T-1) * sum over c != j of cos(k_j, k_c)   (0 for a zero norm),
// the pairwise computation -- O(N^2 b^2) pairs per head -- that the
// Lightning Redundancy Score replaces by pairs inside a block, O(N b^2)
// (nl page "Technische samenvatting", Methodologie item 5; ko page "기술
// 요약", section 2.E).  It exists to measure what that replacement saves;
// the compression itself uses the block-local score.
//
// One workgroup (8 waves) per (request, head).  The inverse norms of all T
// keys go to LDS first.  Then, round by round, every wave holds RB row tiles
// of 16 keys in registers while the workgroup streams the keys in chunks of
// 128 through two LDS buffers (the next chunk's loads are in flight while
// this one is used); each (row tile, column tile) pair is a 16x16 MFMA Gram
// tile, scaled by the column keys' inverse norms and added to per-lane row
// sums, which 16-lane DPP reductions finish.  The diagonal (|k_j|^2 times
// its inverse norm squared, 1 up to rounding) is subtracted as 1.
#include "zp_device.h"
#include "zp_internal.h"
#include "zp_mfma.h"

namespace zp {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 128;        // keys staged in LDS at a time (64 for 512-byte rows)
constexpr int kMaxSlots = kMaxRedundancySlots;  // T bound (inverse norms in LDS)

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of each row of the wave; every lane gets its row's sum.
__device__ inline float row16_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

template <int DT, int D, int B>
__global__ __launch_bounds__(kThreads) void k_redundancy_all(RedundancyParams p) {
  constexpr int EB = Mma<DT>::kElemBytes;
  constexpr int ROWB = D * EB;             // bytes per key row
  constexpr int NV = ROWB / 64;            // 16-byte fragments per lane per row
  constexpr int RB = NV >= 32 ? 1 : 32 / NV;  // row tiles a wave holds (<= 128 registers)
  constexpr int PITCH = ROWB + 16;         // LDS row pitch (breaks bank alignment)
  constexpr int CH = ROWB > 256 ? kChunk / 2 : kChunk;  // keys per chunk (two buffers fit LDS)
  constexpr int PIECES = CH * (ROWB / 16);      // 16-byte pieces of a chunk
  constexpr int PPT = PIECES / kThreads;        // pieces per thread
  static_assert(PIECES % kThreads == 0, "a chunk is whole pieces per thread");
  const int h = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int T = p.n_blocks * B;
  const int32_t* tab = p.tables + (size_t)r * p.n_blocks;
  const char* kbase = static_cast<const char*>(p.k);
  // a table entry outside the pool reads as a zero key (never as memory)
  auto key_ok = [&](int j) -> bool { return (unsigned)tab[j / B] < (unsigned)p.num_blocks; };
  auto key_row = [&](int j) -> const char* {
    const int blk = tab[j / B];
    return kbase + (((size_t)blk * p.H + h) * B + (j % B)) * ROWB;
  };

  __shared__ float s_rinv[kMaxSlots + kChunk];
  __shared__ __attribute__((aligned(16))) char s_k[2][CH * PITCH];  // double buffer

  // inverse norms (0 for a zero key and past the end)
  for (int j = tid; j < T + kChunk; j += kThreads) {
    float rn = 0.f;
    if (j < T && key_ok(j)) {
      const char* row = key_row(j);
      float ss = 0.f;
#pragma unroll
      for (int v = 0; v < ROWB / 16; v++) ss += Mma<DT>::sumsq(ldg16(row + v * 16));
      rn = ss > 0.f ? rsqrtf(ss) : 0.f;
    }
    s_rinv[j] = rn;
  }
  __syncthreads();

  // the 16-byte pieces this thread loads for a chunk starting at slot c0
  auto load_chunk = [&](int c0, uint4 (&pf)[PPT]) {
#pragma unroll
    for (int u = 0; u < PPT; u++) {
      const int x = tid + u * kThreads;
      const int j = c0 + x / (ROWB / 16), piece = x % (ROWB / 16);
      pf[u] = (j < T && key_ok(j)) ? ldg16(key_row(j) + piece * 16) : make_uint4(0, 0, 0, 0);
    }
  };
  const int n_tiles = T / 16;
  const int per_round = kWaves * RB;
  int par = 0;
  for (int t0 = 0; t0 < n_tiles; t0 += per_round) {
    // this wave's row tiles: t0 + wave*RB + k
    uint4 a[RB][NV];
    float acc[RB][4];
#pragma unroll
    for (int k = 0; k < RB; k++) {
      const int rt = t0 + wave * RB + k;
#pragma unroll
      for (int i = 0; i < 4; i++) acc[k][i] = 0.f;
      if (rt < n_tiles && key_ok(rt * 16 + col)) {
        const char* row = key_row(rt * 16 + col) + grp * 16;
#pragma unroll
        for (int v = 0; v < NV; v++) a[k][v] = ldg16(row + v * 64);
      } else {
#pragma unroll
        for (int v = 0; v < NV; v++) a[k][v] = make_uint4(0, 0, 0, 0);
      }
    }
    // Chunks go through two LDS buffers: chunk c is stored into buffer
    // par, then (after one barrier) the loads of chunk c+1 are issued and
    // chunk c is consumed.  Buffer par is next written two chunks later,
    // after a barrier every wave passes only once done with chunk c; the
    // parity runs on across rounds for the same reason.
    uint4 pf[PPT];
    load_chunk(0, pf);
    for (int c0 = 0; c0 < T; c0 += CH, par ^= 1) {
      char* buf = s_k[par];
#pragma unroll
      for (int u = 0; u < PPT; u++) {
        const int x = tid + u * kThreads;
        *reinterpret_cast<uint4*>(buf + (x / (ROWB / 16)) * PITCH + (x % (ROWB / 16)) * 16) = pf[u];
      }
      __syncthreads();
      if (c0 + CH < T) load_chunk(c0 + CH, pf);
      const int nct = min(CH, T - c0) / 16;
      for (int ct = 0; ct < nct; ct++) {
        uint4 bf[NV];
        const char* brow = buf + (ct * 16 + col) * PITCH + grp * 16;
#pragma unroll
        for (int v = 0; v < NV; v++) bf[v] = *reinterpret_cast<const uint4*>(brow + v * 64);
        const float rc = s_rinv[c0 + ct * 16 + col];
#pragma unroll
        for (int k = 0; k < RB; k++) {
          f32x4_t g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int v = 0; v < NV; v++) g = Mma<DT>::step(a[k][v], bf[v], g);
#pragma unroll
          for (int i = 0; i < 4; i++) acc[k][i] = fmaf(g[i], rc, acc[k][i]);
        }
      }
    }
    // finish the row sums and write R_all for this wave's rows
    const float inv_tm1 = 1.0f / (float)(T - 1);
#pragma unroll
    for (int k = 0; k < RB; k++) {
      const int rt = t0 + wave * RB + k;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float sum = row16_sum(acc[k][i]);
        const int j = rt * 16 + 4 * grp + i;
        if (rt < n_tiles && col == 0) {
          const float ra = s_rinv[j];
          p.out[((size_t)r * p.H + h) * T + j] = ra > 0.f ? (ra * sum - 1.0f) * inv_tm1 : 0.f;
        }
      }
    }
  }
}

template <int DT, int D>
hipError_t launch_d(const RedundancyParams& p, int block_size, hipStream_t s) {
  const dim3 grid(p.H, p.R);
  if (block_size == 16)
    hipLaunchKernelGGL((k_redundancy_all<DT, D, 16>), grid, dim3(kThreads), 0, s, p);
  else if (block_size == 32)
    hipLaunchKernelGGL((k_redundancy_all<DT, D, 32>), grid, dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const RedundancyParams& p, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 64) return launch_d<DT, 64>(p, block_size, s);
  if (head_dim == 128) return launch_d<DT, 128>(p, block_size, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_redundancy_all(const RedundancyParams& p, int dtype, int head_dim,
                                 int block_size, hipStream_t s) {
  if (p.R <= 0) return hipSuccess;
  if (p.n_blocks * block_size > kMaxSlots || p.n_blocks * block_size < 2) return hipErrorInvalidValue;
  prof_begin(ZP_PHASE_REDUNDANCY_ALL, s);
  hipError_t e = dtype == ZP_BF16 ? launch_dt<ZP_BF16>(p, head_dim, block_size, s)
                 : dtype == ZP_F32 ? launch_dt<ZP_F32>(p, head_dim, block_size, s)
                                   : hipErrorInvalidValue;
  prof_end(ZP_PHASE_REDUNDANCY_ALL, s);
  return e;
}

}  // namespace zp
