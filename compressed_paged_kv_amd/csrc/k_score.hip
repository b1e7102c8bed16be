// Scoring kernels of the compression pass (gfx950).
//
// For one (layer, request, KV head) "unit" the observation window supplies
// rows = G*w query rows (G query heads of the group times the w window
// positions; ko page section 2.A).  Every cached slot j gets
//   A[j] = mean over rows of the causal softmax of q.k_j / sqrt(d),
//   R[j] = mean cosine of k_j with the other keys of its block (Lightning
//          Redundancy Score, nl page Methodologie item 5 / ko page 2.E),
//   s[j] = A[j] * (1 - R[j]) for the candidates j < T - w.
// The softmax needs each row's max and normaliser over all T slots before
// any probability can be summed over rows, so the pass runs twice over K:
//   k_score_stats: per token chunk, running (max, sum) of every row;
//   k_score_final: merges the chunk statistics, recomputes the logits and
//                  accumulates A, computes the in-block Gram for R, writes s.
// Both contractions (rows x b logits, b x b Gram) are 16x16 MFMA tiles:
// v_mfma_f32_16x16x32_bf16 for bfloat16 caches, v_mfma_f32_16x16x4f32 for
// float32 ones.  A lane holds operand row (lane % 16) and a 16-byte slice of
// the head dimension chosen by lane / 16; the output tile gives lane
// rows 4*(lane/16)+i, column lane % 16.  Q and K use the same slicing, so the
// contraction over the head dimension is exact whatever order the hardware
// sums the slices in.
#include "zp_device.h"
#include "zp_internal.h"

namespace zp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kInitMax = -1.0e30f;  // finite "minus infinity" so merges never form inf - inf
constexpr float kLazy = 8.0f;         // rescale the running sum only when the max grows by > 2^8

template <int DT>
struct Mma;

template <>
struct Mma<ZP_BF16> {
  static constexpr int kElemBytes = 2;
  __device__ static inline f32x4_t step(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static inline float sumsq(uint4 a) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float lo = __uint_as_float(w[k] << 16);
      float hi = __uint_as_float(w[k] & 0xFFFF0000u);
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
    return s;
  }
};

template <>
struct Mma<ZP_F32> {
  static constexpr int kElemBytes = 4;
  __device__ static inline f32x4_t step(uint4 a, uint4 b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
  __device__ static inline float sumsq(uint4 a) {
    float x = __uint_as_float(a.x), y = __uint_as_float(a.y);
    float z = __uint_as_float(a.z), w = __uint_as_float(a.w);
    return fmaf(w, w, fmaf(z, z, fmaf(y, y, x * x)));
  }
};

__device__ inline uint4 ld16(const char* p) { return ldg16(p); }

// 2^x on the hardware unit (results below 2^-126 flush to zero).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two (max, sum) pairs that represent sum_k 2^(x_k - max).
__device__ inline void merge_stat(float& m, float& z, float m2, float z2) {
  float M = fmaxf(m, m2);
  z = z * fast_exp2(m - M) + z2 * fast_exp2(m2 - M);
  m = M;
}

// Physical id of block blk0 + wave + 4*i is held by lane i (i < 64); the
// wave's block list is read once instead of once per block.
__device__ inline int wave_block_ids(const ScoreParams& p, int r, int blk0, int blk1, int wave,
                                     int lane) {
  const int n = blk0 + wave + 4 * lane;
  return n < blk1 ? p.src[(size_t)r * p.n_max + n] : 0;
}

// Query fragments of the unit's rows: row = i*G + g holds window position i
// of query head h*G + g.  Rows beyond `rows` are zero.
template <int DT, int D, int RT>
__device__ inline void load_q(const ScoreParams& p, const char* qbase, int r, int h, int col,
                              int grp, uint4 (&qf)[RT][D * Mma<DT>::kElemBytes / 64]) {
  constexpr int EB = Mma<DT>::kElemBytes;
  constexpr int NV = D * EB / 64;
#pragma unroll
  for (int rt = 0; rt < RT; rt++) {
    const int row = rt * 16 + col;
    if (row < p.rows) {
      const int i = row / p.G, g = row - i * p.G;
      const char* ptr = qbase + ((size_t)(r * p.w + i) * p.Hq + (size_t)h * p.G + g) * D * EB + grp * 16;
#pragma unroll
      for (int v = 0; v < NV; v++) qf[rt][v] = ld16(ptr + v * 64);
    } else {
#pragma unroll
      for (int v = 0; v < NV; v++) qf[rt][v] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Last slot each of the lane's output rows may attend to (causal window),
// -1 for padding rows.
template <int RT>
__device__ inline void row_limits(const ScoreParams& p, int grp, int (&lim)[RT][4]) {
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = rt * 16 + 4 * grp + i;
      lim[rt][i] = row < p.rows ? p.T - p.w + row / p.G : -1;
    }
}

template <int DT, int D, int B, int RT>
__global__ __launch_bounds__(256) void k_score_stats(ScoreParams p) {
  constexpr int EB = Mma<DT>::kElemBytes;
  constexpr int NV = D * EB / 64;
  constexpr int NST = B / 16;
  constexpr int RP = RT * 16;
  const int chunk = blockIdx.x, h = blockIdx.y, lr = blockIdx.z;
  const int l = lr / p.R, r = lr - l * p.R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const char* kbase = static_cast<const char*>(p.layer_ptrs[l * kPtrsPerLayer + 0]);
  const char* qbase = static_cast<const char*>(p.layer_ptrs[l * kPtrsPerLayer + 2]);

  uint4 qf[RT][NV];
  load_q<DT, D, RT>(p, qbase, r, h, col, grp, qf);
  int lim[RT][4];
  row_limits<RT>(p, grp, lim);
  float m[RT][4], z[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int i = 0; i < 4; i++) { m[rt][i] = kInitMax; z[rt][i] = 0.f; }

  const int blk0 = chunk * p.chunk_blocks;
  const int blk1 = min(blk0 + p.chunk_blocks, p.n_max);
  const int n_items = blk1 - blk0 - wave > 0 ? (blk1 - blk0 - wave + 3) / 4 : 0;
  const int ids = wave_block_ids(p, r, blk0, blk1, wave, lane);
  const int row_off = col * D * EB + grp * 16;
  // K fragments of the wave's next block are loaded (unconditionally, the
  // last block again at the end) while the current one is consumed
  auto fetch = [&](int i, uint4 (&kf)[NST][NV]) {
    const int pblk = __builtin_amdgcn_readlane(ids, min(i, n_items - 1));
    const char* tile = kbase + ((size_t)pblk * p.H + h) * B * D * EB + row_off;
#pragma unroll
    for (int st = 0; st < NST; st++)
#pragma unroll
      for (int v = 0; v < NV; v++) kf[st][v] = ld16(tile + st * 16 * D * EB + v * 64);
  };
  uint4 kcur[NST][NV], knext[NST][NV];
  if (n_items > 0) fetch(0, kcur);
  for (int it = 0; it < n_items; it++) {
    fetch(it + 1, knext);
    const int n = blk0 + wave + 4 * it;
#pragma unroll
    for (int st = 0; st < NST; st++) {
      const int j = n * B + st * 16 + col;
#pragma unroll
      for (int rt = 0; rt < RT; rt++) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; v++) acc = Mma<DT>::step(qf[rt][v], kcur[st][v], acc);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if (j <= lim[rt][i]) {
            const float x = acc[i] * p.scale_log2;
            const bool up = x > m[rt][i] + kLazy;
            const float t = fast_exp2(up ? m[rt][i] - x : x - m[rt][i]);
            z[rt][i] = up ? fmaf(z[rt][i], t, 1.f) : z[rt][i] + t;
            m[rt][i] = up ? x : m[rt][i];
          }
        }
      }
    }
#pragma unroll
    for (int st = 0; st < NST; st++)
#pragma unroll
      for (int v = 0; v < NV; v++) kcur[st][v] = knext[st][v];
  }
  // merge the 16 columns of every row
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float m2 = __shfl_xor(m[rt][i], off);
        const float z2 = __shfl_xor(z[rt][i], off);
        merge_stat(m[rt][i], z[rt][i], m2, z2);
      }
  __shared__ float sm[4][RP][2];
  if (col == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        sm[wave][rt * 16 + 4 * grp + i][0] = m[rt][i];
        sm[wave][rt * 16 + 4 * grp + i][1] = z[rt][i];
      }
  }
  __syncthreads();
  if (threadIdx.x < RP) {
    const int row = threadIdx.x;
    float M = sm[0][row][0], Z = sm[0][row][1];
    for (int wv = 1; wv < 4; wv++) merge_stat(M, Z, sm[wv][row][0], sm[wv][row][1]);
    const size_t unit = (size_t)lr * p.H + h;
    float* out = p.stats + ((unit * p.nchunk + chunk) * p.rows_pad + row) * 2;
    out[0] = M;
    out[1] = Z;
  }
}

template <int DT, int D, int B, int RT>
__global__ __launch_bounds__(256) void k_score_final(ScoreParams p) {
  constexpr int EB = Mma<DT>::kElemBytes;
  constexpr int NV = D * EB / 64;
  constexpr int NST = B / 16;
  constexpr int RP = RT * 16;
  // Workgroups run in the reverse order of the statistics pass, so the keys
  // read last by that pass (most likely still in the last-level cache) are
  // read again first.
  const int chunk = gridDim.x - 1 - blockIdx.x, h = gridDim.y - 1 - blockIdx.y;
  const int lr = gridDim.z - 1 - blockIdx.z;
  const int l = lr / p.R, r = lr - l * p.R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const size_t unit = (size_t)lr * p.H + h;
  const char* kbase = static_cast<const char*>(p.layer_ptrs[l * kPtrsPerLayer + 0]);
  const char* qbase = static_cast<const char*>(p.layer_ptrs[l * kPtrsPerLayer + 2]);

  // final (max, 1/sum) of every row from the chunk statistics
  __shared__ float smz[RP][2];
  if (threadIdx.x < RP) {
    const int row = threadIdx.x;
    const float* st = p.stats + (unit * p.nchunk * p.rows_pad + row) * 2;
    float M = kInitMax, Z = 0.f;
    for (int c = 0; c < p.nchunk; c++)
      merge_stat(M, Z, st[(size_t)c * p.rows_pad * 2], st[(size_t)c * p.rows_pad * 2 + 1]);
    smz[row][0] = M;
    smz[row][1] = Z > 0.f ? 1.0f / Z : 0.f;
  }
  __syncthreads();
  float rm[RT][4], rz[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      rm[rt][i] = smz[rt * 16 + 4 * grp + i][0];
      rz[rt][i] = smz[rt * 16 + 4 * grp + i][1];
    }
  uint4 qf[RT][NV];
  load_q<DT, D, RT>(p, qbase, r, h, col, grp, qf);
  int lim[RT][4];
  row_limits<RT>(p, grp, lim);
  const float inv_rows = 1.0f / (float)p.rows;
  const float inv_bm1 = 1.0f / (float)(B - 1);

  const int blk0 = chunk * p.chunk_blocks;
  const int blk1 = min(blk0 + p.chunk_blocks, p.n_max);
  const int n_items = blk1 - blk0 - wave > 0 ? (blk1 - blk0 - wave + 3) / 4 : 0;
  const int ids = wave_block_ids(p, r, blk0, blk1, wave, lane);
  const int row_off = col * D * EB + grp * 16;
  auto fetch = [&](int i, uint4 (&kd)[NST][NV]) {
    const int pblk = __builtin_amdgcn_readlane(ids, min(i, n_items - 1));
    const char* tile = kbase + ((size_t)pblk * p.H + h) * B * D * EB + row_off;
#pragma unroll
    for (int st = 0; st < NST; st++)
#pragma unroll
      for (int v = 0; v < NV; v++) kd[st][v] = ld16(tile + st * 16 * D * EB + v * 64);
  };
  uint4 kf[NST][NV], knext[NST][NV];
  if (n_items > 0) fetch(0, kf);
  for (int it = 0; it < n_items; it++) {
    fetch(it + 1, knext);
    const int n = blk0 + wave + 4 * it;
    float A[NST], Rd[NST], nrm[NST];
#pragma unroll
    for (int st = 0; st < NST; st++) {
      // importance: column sums of the row probabilities, fixed order
      const int j = n * B + st * 16 + col;
      float cs = 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; rt++) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; v++) acc = Mma<DT>::step(qf[rt][v], kf[st][v], acc);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float pr = fast_exp2(acc[i] * p.scale_log2 - rm[rt][i]) * rz[rt][i];
          cs += (j <= lim[rt][i]) ? pr : 0.f;
        }
      }
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      A[st] = cs * inv_rows;
      // squared norm of key (st*16 + col)
      float ss = 0.f;
#pragma unroll
      for (int v = 0; v < NV; v++) ss += Mma<DT>::sumsq(kf[st][v]);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      nrm[st] = ss;
    }
    // redundancy: column sums of the in-block cosine matrix, diagonal excluded.
    // Inverse norms of the lane's output rows (key 4*grp+i of sub-tile s1)
    // come from the lane that holds that key as its column.
    float ra[NST][4];
#pragma unroll
    for (int s1 = 0; s1 < NST; s1++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float na = __shfl(nrm[s1], 4 * grp + i);
        ra[s1][i] = na > 0.f ? rsqrtf(na) : 0.f;
      }
#pragma unroll
    for (int s2 = 0; s2 < NST; s2++) {
      float cs = 0.f;
      const float nc = nrm[s2];
      const float rc = nc > 0.f ? rsqrtf(nc) : 0.f;
#pragma unroll
      for (int s1 = 0; s1 < NST; s1++) {
        f32x4_t g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; v++) g = Mma<DT>::step(kf[s1][v], kf[s2][v], g);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const bool diag = (s1 == s2) && (4 * grp + i == col);
          cs += diag ? 0.f : g[i] * ra[s1][i] * rc;
        }
      }
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      Rd[s2] = cs * inv_bm1;
    }
    if (grp == 0) {
#pragma unroll
      for (int st = 0; st < NST; st++) {
        const int j = n * B + st * 16 + col;
        const float s = A[st] * (1.0f - Rd[st]);
        const size_t o = unit * p.T + j;
        p.score[o] = s;
        if (p.dbg_importance) p.dbg_importance[o] = A[st];
        if (p.dbg_redundancy) p.dbg_redundancy[o] = Rd[st];
        if (p.dbg_score && j < p.C) p.dbg_score[o] = s;
      }
    }
#pragma unroll
    for (int st = 0; st < NST; st++)
#pragma unroll
      for (int v = 0; v < NV; v++) kf[st][v] = knext[st][v];
  }
}

template <int DT, int D, int B, int RT>
hipError_t launch_rt(const ScoreParams& p, int units, hipStream_t s) {
  dim3 grid(p.nchunk, p.H, units / p.H);
  prof_begin(ZP_PHASE_SCORE_STATS, s);
  hipLaunchKernelGGL((k_score_stats<DT, D, B, RT>), grid, dim3(256), 0, s, p);
  prof_end(ZP_PHASE_SCORE_STATS, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(ZP_PHASE_SCORE, s);
  hipLaunchKernelGGL((k_score_final<DT, D, B, RT>), grid, dim3(256), 0, s, p);
  prof_end(ZP_PHASE_SCORE, s);
  return hipGetLastError();
}

template <int DT, int D, int B>
hipError_t launch_b(const ScoreParams& p, int units, hipStream_t s) {
  switch (p.rows_pad / 16) {
    case 1: return launch_rt<DT, D, B, 1>(p, units, s);
    case 2: return launch_rt<DT, D, B, 2>(p, units, s);
    case 4: return launch_rt<DT, D, B, 4>(p, units, s);
    case 8: return launch_rt<DT, D, B, 8>(p, units, s);
  }
  return hipErrorInvalidValue;
}

template <int DT, int D>
hipError_t launch_d(const ScoreParams& p, int block_size, int units, hipStream_t s) {
  if (block_size == 16) return launch_b<DT, D, 16>(p, units, s);
  if (block_size == 32) return launch_b<DT, D, 32>(p, units, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const ScoreParams& p, int head_dim, int block_size, int units, hipStream_t s) {
  if (head_dim == 64) return launch_d<DT, 64>(p, block_size, units, s);
  if (head_dim == 128) return launch_d<DT, 128>(p, block_size, units, s);
  return hipErrorInvalidValue;
}

}  // namespace

int score_row_tiles(int rows) {
  if (rows <= 0 || rows > kMaxScoreRows) return 0;
  int t = (rows + 15) / 16;
  int p2 = 1;
  while (p2 < t) p2 <<= 1;
  return p2;
}

hipError_t launch_score(const ScoreParams& p, int dtype, int head_dim, int block_size, int units,
                        hipStream_t s) {
  if (units <= 0) return hipSuccess;
  if (dtype == ZP_BF16) return launch_dt<ZP_BF16>(p, head_dim, block_size, units, s);
  if (dtype == ZP_F32) return launch_dt<ZP_F32>(p, head_dim, block_size, units, s);
  return hipErrorInvalidValue;
}

}  // namespace zp
