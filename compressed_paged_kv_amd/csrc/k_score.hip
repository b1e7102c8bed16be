// Scoring and survivor selection of the compression pass (gfx950).
//
// One workgroup (four waves, or eight with two row groups) per (layer,
// request, KV head) "unit".  The
// observation window supplies rows = G*w query rows (the G query heads of
// the group times the w window positions; ko page section 2.A).  Every
// cached slot j gets
//   A[j] = mean over rows of the causal softmax of q.k_j / sqrt(d),
//   R[j] = mean cosine of k_j with the other keys of its block (Lightning
//          Redundancy Score, nl page Methodologie item 5 / ko page 2.E),
//   s[j] = A[j] * (1 - R[j]) for the candidates j < C = T - w,
// and the E = T - K_keep candidates with the smallest (s, then highest
// slot) are evicted; the window slots always stay.
//
// Phases, all inside the workgroup:
//   1. softmax statistics: each wave runs over its share of the unit's
//      blocks keeping, per window row, a running (max, sum of 2^(x - max))
//      that is rescaled only when the max grows by more than 64 (log2
//      units); lanes and waves are then merged in LDS into one exponent
//      offset per row, M + log2(Z), so a probability is a single
//      2^(x - offset)
//      (skipped when the caller supplies each window row's log-sum-exp);
//   2. the same blocks again, in reverse order so the first ones are those
//      pass 1 read last, still in cache: probabilities summed over the
//      rows in a fixed order (so equal inputs give bit-equal importances),
//      the in-block Gram matrix for the cosines, and s into LDS;
//   3. the selection (select_evicted): radix passes over order-preserving
//      32-bit keys, starting below the prefix all keys share, narrow the bin
//      of the E-th smallest score; a small bin is ranked exactly, a large
//      bin of equal keys gives up its highest slots; one prefix sum in slot
//      order places the ascending evicted list;
//   4. (k_score_compact) the in-place compaction of the unit's K and V
//      rows (compact_unit).
// A request may hold more blocks than the cap, its own number when table
// rows are padded with -1; its window rows are its own or, with query
// slots, those of its slot in the decode's query store.
// The rows x b logit tiles and the b x b Gram tiles are 16x16 MFMA tiles:
// v_mfma_f32_16x16x32_bf16 for bfloat16 caches, v_mfma_f32_16x16x4f32 for
// float32 ones.  A lane holds operand row (lane % 16) and a 16-byte slice of
// the head dimension chosen by lane / 16; the output tile gives lane rows
// 4*(lane/16)+i, column lane % 16.  Q and K use the same slicing, so the
// contraction over the head dimension is exact whatever order the hardware
// sums the slices in.  With more than 64 rows the waves split into two row
// groups whose partial importances are added once both are done.
#include "zp_device.h"
#include "zp_internal.h"
#include "zp_mfma.h"

namespace zp {
namespace {


// Waves per workgroup: four with one row group (two workgroups share a CU;
// with more units than workgroup slots one selects while another streams
// K); eight with two row groups, whose paired waves exchange K tiles
// through LDS, each pair synchronising on its own.
template <int RG>
constexpr int score_waves() { return RG == 2 ? 8 : 4; }
constexpr int kMaxWaves = 8;
constexpr float kInitMax = -1.0e30f;  // finite "minus infinity": merges never form inf - inf
// A running sum is rescaled only when a term would exceed 2^kLazy: terms stay
// below 2^64 and a sum of at most 8192 of them below 2^77, far from the float
// range, while a lane that saw one low logit first (it holds one key per
// block) rarely has to leave the fast path.
constexpr float kLazy = 64.0f;
constexpr float kLazyTerm = 18446744073709551616.0f;  // 2^kLazy
constexpr float kMasked = -3.0e38f;   // logit of a causally masked slot: adds 2^(-huge) = 0
// scores (T <= 8192) with one row group; three T <= 4096 arrays with two
template <int RG>
constexpr int lds_floats() { return RG == 2 ? 3 * 4096 : 8192; }
// Registers per lane for the K ring (blocks loaded ahead of the one being
// scored).  One row group: 64, so four 4 KiB (block, head) tiles of a
// b = 16, d = 128 bfloat16 cache are in flight per wave -- keys that come
// cold from HBM need the depth, cached ones do not.  Two row groups (the
// b = 32, 128-row shape, bound by issue rather than by loads): 32.
#ifndef ZP_SCORE_RING_VGPRS
#define ZP_SCORE_RING_VGPRS 64
#endif
#ifndef ZP_SCORE_RING_VGPRS_2RG
#define ZP_SCORE_RING_VGPRS_2RG 32
#endif
#ifndef ZP_SCORE_REVERSE
#define ZP_SCORE_REVERSE 1
#endif
constexpr bool kReversePass2 = ZP_SCORE_REVERSE != 0;
#ifndef ZP_FUSED_UNROLL
#define ZP_FUSED_UNROLL 6
#endif
constexpr int kFusedUnroll = ZP_FUSED_UNROLL;  // rows per thread per tile of the fused compaction

template <bool V>
struct BoolC {
  static constexpr bool value = V;
};


__device__ inline uint4 ld16(const char* p) { return ldg16(p); }

// 2^x and log2(x) on the hardware unit (2^x below 2^-126 flushes to zero).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <int CTRL>
__device__ inline float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the four 16-lane rows: every lane gets ((row0 + row1) + (row2 +
// row3)) for its column, in the same order for every column.
__device__ inline float sum_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Merge two (max, sum) pairs that represent sum_k 2^(x_k - max).
__device__ inline void merge_stat(float& m, float& z, float m2, float z2) {
  const float M = fmaxf(m, m2);
  z = z * fast_exp2(m - M) + z2 * fast_exp2(m2 - M);
  m = M;
}

template <int CTRL>
__device__ inline void merge_dpp(float& m, float& z) {
  const float m2 = dpp<CTRL>(m), z2 = dpp<CTRL>(z);
  merge_stat(m, z, m2, z2);
}

// Running statistics update for one logit x (log2 units).
__device__ inline void lazy_update(float& m, float& z, float x) {
  const bool up = x > m + kLazy;
  const float t = fast_exp2(up ? m - x : x - m);
  z = up ? fmaf(z, t, 1.f) : z + t;
  m = up ? x : m;
}

__device__ inline uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);  // -0 + 0 = +0 under round-to-nearest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive workgroup-wide sum; `scratch` holds >= NW ints.  Ends with
// a barrier so scratch may be reused.
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

// Minimum over the wave: DPP inside 16-lane rows, then the row swaps.
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
__device__ inline uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = min(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = min(x, dpp_u32<0x141>(x));  // row_half_mirror
  x = min(x, dpp_u32<0x140>(x));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = min(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return min(b[0], b[1]);
}

// Selection state in LDS.  Histograms are triple-buffered: pass p counts
// into buffer p % 3 and clears buffer (p + 1) % 3, which every wave finished
// scanning before the barrier of pass p - 1, so each pass needs a single
// barrier.  Small target bins are resolved in `list`.
constexpr int kSelList = 64;
struct SelectLds {
  int hist[3][256];
  unsigned long long list[kSelList];  // (key << 32) | ~slot of the target bin's candidates
  uint32_t evict_bits[kMaxScoreSlots / 32];
  uint32_t wave_min[kMaxWaves], wave_max[kMaxWaves];
  int count;
};

// Evicts the E candidates (slots j < C) with the smallest order keys, equal
// keys taking the higher slot first, and writes them ascending.  Thread t
// owns the contiguous slots [t*per, t*per + per); PER >= per.
//   1. The block's smallest and largest key share a prefix, which the
//      E-th smallest key shares too.
//   2. Radix passes of up to 8 bits below the known prefix narrow the
//      bin that holds the E-th smallest key; every wave reads the histogram
//      and finds the bin itself (4 bins a lane, one wave-wide scan).
//   3. Once that bin holds at most kSelList keys, each of them is ranked
//      against the others by (key, higher slot first) and the first `rank`
//      are marked; if all 32 bits are fixed and the bin is still larger,
//      its keys are all equal and the highest `rank` slots of them go.
//   4. One workgroup prefix sum gives every thread its output position.
// s_f (LDS, may be null) also gets f_i = e_i - i for the i-th evicted slot.
template <int PER, int NW>
__device__ inline void select_evicted(const float* s_sc, SelectLds& L, int* s_scr,
                                      const ScoreParams& p, size_t unit, int* s_f, const int T,
                                      const int C, const int E) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (T + 64 * NW - 1) / (64 * NW);
  const int j0 = tid * per;
  uint32_t key[PER];
  if (per == PER) {  // 16-byte groups; a range past T stays inside s_buf (threads * PER floats)
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(s_sc + j0 + i);
      key[i] = order_key(v.x);
      key[i + 1] = order_key(v.y);
      key[i + 2] = order_key(v.z);
      key[i + 3] = order_key(v.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; i++) key[i] = (i < per && j0 + i < T) ? order_key(s_sc[j0 + i]) : 0u;
  }
  auto valid = [&](int i) { return i < per && j0 + i < C; };
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < PER; i++)
    if (valid(i)) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  for (int t = tid; t < 256; t += 64 * NW) L.hist[0][t] = 0;
  for (int t = tid; t < kMaxScoreSlots / 32; t += 64 * NW) L.evict_bits[t] = 0u;
  if (tid == 0) L.count = 0;
  kmin = wave_min_u32(kmin);
  kmax = ~wave_min_u32(~kmax);
  if (lane == 0) {
    L.wave_min[wave] = kmin;
    L.wave_max[wave] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; w++) {
    kmin = min(kmin, L.wave_min[w]);
    kmax = max(kmax, L.wave_max[w]);
  }
  const uint32_t diff = kmin ^ kmax;
  int done = diff ? __clz((int)diff) : 32;  // leading bits every candidate key shares
  uint32_t mask = done == 0 ? 0u : done == 32 ? 0xFFFFFFFFu : 0xFFFFFFFFu << (32 - done);
  uint32_t prefix = kmin & mask;
  int rank = E;     // the E-th smallest key is the rank-th smallest of the bin
  int cnt = C;      // candidates in the bin
  int pass = 0;
  while (cnt > kSelList && done < 32) {
    const int nb = min(8, 32 - done), shift = 32 - done - nb;
    int* h = L.hist[pass % 3];
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (valid(i) && (key[i] & mask) == prefix) atomicAdd(&h[(key[i] >> shift) & ((1u << nb) - 1u)], 1);
    for (int t = tid; t < 256; t += 64 * NW) L.hist[(pass + 1) % 3][t] = 0;
    __syncthreads();
    const int4 hv = *reinterpret_cast<const int4*>(&h[lane * 4]);
    const int c4 = hv.x + hv.y + hv.z + hv.w;
    int incl = c4;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int excl = incl - c4;
    const unsigned long long hit = __ballot(excl < rank && incl >= rank);
    const int src = hit ? __builtin_ctzll(hit) : 0;
    int sb = 0, below = excl, cb = hv.x;
    if (below + hv.x < rank) {
      below += hv.x; sb = 1; cb = hv.y;
      if (below + hv.y < rank) {
        below += hv.y; sb = 2; cb = hv.z;
        if (below + hv.z < rank) { below += hv.z; sb = 3; cb = hv.w; }
      }
    }
    const uint32_t bin = (uint32_t)__builtin_amdgcn_readlane(lane * 4 + sb, src);
    rank -= __builtin_amdgcn_readlane(below, src);
    cnt = __builtin_amdgcn_readlane(cb, src);
    prefix |= bin << shift;
    mask |= ((1u << nb) - 1u) << shift;
    done += nb;
    pass++;
  }
  const bool listed = cnt <= kSelList;
  if (listed) {
    // the bin's candidates into the list: one atomic per wave
    int mine = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) mine += (valid(i) && (key[i] & mask) == prefix) ? 1 : 0;
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    int base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&L.count, incl);
    base = __shfl(base, 63) + incl - mine;
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (valid(i) && (key[i] & mask) == prefix) {
        if (base < kSelList)
          L.list[base] = ((unsigned long long)key[i] << 32) | (uint32_t)(~(uint32_t)(j0 + i));
        base++;
      }
    __syncthreads();
    if (tid < cnt) {
      const unsigned long long me = L.list[tid];
      int below = 0;
      for (int u = 0; u < cnt; u++) below += L.list[u] < me ? 1 : 0;
      if (below < rank) {
        const uint32_t j = ~(uint32_t)me;
        atomicOr(&L.evict_bits[j >> 5], 1u << (j & 31));
      }
    }
    __syncthreads();
  }
  // per thread: evicted slots decided so far, and (equal-key case) the
  // keys equal to the bin's key, packed in one prefix sum
  int sure = 0, ties = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    if (!valid(i)) continue;
    if (key[i] < prefix) {
      sure++;
    } else if ((key[i] & mask) == prefix) {
      const int j = j0 + i;
      if (listed) sure += (L.evict_bits[j >> 5] >> (j & 31)) & 1u;
      else ties++;
    }
  }
  const int packed = sure | (ties << 16);  // both sums stay below 2^16 (T <= 8192)
  const int excl = block_incl_sum(packed, s_scr) - packed;
  const int tie_from = cnt - rank;  // tie index (slot order) from which equal keys go
  int tie_idx = excl >> 16;
  int pos = (excl & 0xFFFF) + (listed ? 0 : max(0, tie_idx - tie_from));
  int kept_pos = j0 - pos;  // survivors below j0
  int32_t* out = p.evicted + unit * p.E;   // stride: the call's largest E
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int j = j0 + i;
    if (i >= per || j >= T) continue;
    bool ev = false;
    if (j < C) {
      if (key[i] < prefix) {
        ev = true;
      } else if ((key[i] & mask) == prefix) {
        if (listed) {
          ev = (L.evict_bits[j >> 5] >> (j & 31)) & 1u;
        } else {
          ev = tie_idx >= tie_from;
          tie_idx++;
        }
      }
    }
    if (ev) {
      if (pos < E) {
        out[pos] = j;
        if (s_f) s_f[pos] = j - pos;
      }
      pos++;
    } else {
      if (p.dbg_kept && kept_pos >= 0 && kept_pos < p.K_keep) p.dbg_kept[unit * p.K_keep + kept_pos] = j;
      kept_pos++;
    }
  }
}

// Compaction of one (layer, request, head) unit right after its selection,
// by the workgroup that scored it: logical slot r < K_keep of the target
// blocks receives old slot kept[r], for K and V, with kept rebuilt from the
// evicted list as kept[r] = r + #{i : f_i <= r}, f_i = e_i - i (nl page
// Methodologie item 1, ko page section 2.C: survivors move in order into the
// first N_max-1 blocks; shared sources are never written).
//
// Units never touch each other's rows: a unit writes only rows of its own
// head and layer, in blocks private to its request or freshly allocated, and
// every other unit reads other heads, layers or requests.  Inside the unit
// the in-place rule of the standalone compaction holds: target slot r is old
// slot r or a fresh block, old slot r is read only by rows r' <= r, and the
// workgroup walks ascending tiles whose loads all return before the barrier
// and whose stores all come after it.  Rows below the first evicted slot and
// the first re-targeted block stay where they are.
//
// LDS (inside the score array, free once the keys are in registers): f from
// the selection, then kept, and the request's source and target block ids.
template <int VPR, int B, int NTH, int U, bool KCACHED>
__device__ inline void compact_unit(const ScoreParams& p, float* lds, int* s_first, int l, int r,
                                    int h, const int n_src, const int E) {
  constexpr int kRowsPerPass = NTH / VPR;
  constexpr int kRowsPerTile = kRowsPerPass * U;
  constexpr size_t kRowBytes = (size_t)VPR * 16;
  const int tid = threadIdx.x;
  const int vec = tid % VPR, rsub = tid / VPR;
  const int* f = reinterpret_cast<const int*>(lds);
  unsigned short* kept = reinterpret_cast<unsigned short*>(lds + kMaxEvicted);
  int* srcb = reinterpret_cast<int*>(lds + kMaxEvicted + kMaxScoreSlots / 2);
  int* dstb = srcb + kMaxScoreSlots / 16;
  // an id outside the pool is read as block 0 and never written
  for (int n = tid; n < n_src; n += NTH) {
    const int id = p.src[(size_t)r * p.src_stride + n];
    srcb[n] = (unsigned)id < (unsigned)p.num_blocks ? id : 0;
  }
  for (int n = tid; n < p.n_max - 1; n += NTH) {
    const int id = p.dst[(size_t)r * p.dst_stride + n];
    dstb[n] = (unsigned)id < (unsigned)p.num_blocks ? id : -1;
  }
  if (tid == 0) *s_first = p.K_keep;
  __syncthreads();  // f (written by the selection) and the block ids are in LDS
  // the first re-targeted block (a new block for a shared source) ...
  for (int n = tid; n < p.n_max - 1; n += NTH)
    if (dstb[n] != srcb[n]) atomicMin(s_first, n * B);
  for (int row = tid; row < p.K_keep; row += NTH) {
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (f[mid] <= row) lo = mid + 1; else hi = mid;
    }
    kept[row] = (unsigned short)(row + lo);
  }
  __syncthreads();
  // ... and the first evicted slot (f_0 = e_0): nothing below both moves
  const int first = min(min(*s_first, E > 0 ? f[0] : p.K_keep), p.K_keep);
  if (first >= p.K_keep) return;  // nothing moves (uniform)

  char* const kbase = static_cast<char*>(p.layers[l - p.layer0].k) + vec * 16;
  char* const vbase = static_cast<char*>(p.layers[l - p.layer0].v) + vec * 16;
  auto row_of = [&](int blk, int off) -> int { return (blk * p.H + h) * B + off; };
  auto off_of = [&](int row) -> size_t { return (size_t)(unsigned)row * kRowBytes; };
  // Rows past the end are clamped to the last row; unmoved rows are read
  // but not written (target -1).  V rows are streamed both ways.  K rows
  // are loaded and stored normally (KCACHED) when every unit of the call is
  // resident at once: the scoring has just read them and many are still
  // cached, and the decode that follows finds some of the stored rows
  // there.  With several rounds of workgroups, normal accesses only crowd
  // out what the later rounds' scoring reads, and K is streamed too.
  auto load_tile = [&](int t0, uint4 (&kb)[U], uint4 (&vb)[U], int (&to)[U]) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int row = min(t0 + rsub + u * kRowsPerPass, p.K_keep - 1);
      const int j = kept[row];
      const int from = row_of(srcb[j / B], j % B);
      const int db = dstb[row / B];
      const int dst = row_of(db, row % B);
      kb[u] = KCACHED ? ldg16(kbase + off_of(from)) : ldg16_stream(kbase + off_of(from));
      vb[u] = ldg16_stream(vbase + off_of(from));
      to[u] = (db >= 0 && dst != from && t0 + rsub + u * kRowsPerPass < p.K_keep) ? dst : -1;
    }
  };
  uint4 ck[U], cv[U], nk[U], nv[U];
  int cto[U], nto[U];
  load_tile(first, ck, cv, cto);
  for (int t0 = first; t0 < p.K_keep; t0 += kRowsPerTile) {
    load_tile(min(t0 + kRowsPerTile, p.K_keep - 1), nk, nv, nto);
    // every load of this tile has returned before any thread stores
#pragma unroll
    for (int u = 0; u < U; u++) {
      asm volatile("" ::"v"(ck[u].x), "v"(ck[u].y), "v"(ck[u].z), "v"(ck[u].w));
      asm volatile("" ::"v"(cv[u].x), "v"(cv[u].y), "v"(cv[u].z), "v"(cv[u].w));
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; u++)
      if (cto[u] >= 0) {
        if constexpr (KCACHED) stg16(kbase + off_of(cto[u]), ck[u]);
        else stg16_stream(kbase + off_of(cto[u]), ck[u]);
        stg16_stream(vbase + off_of(cto[u]), cv[u]);
      }
#pragma unroll
    for (int u = 0; u < U; u++) {
      ck[u] = nk[u];
      cv[u] = nv[u];
      cto[u] = nto[u];
    }
  }
}

// Workgroups a CU is to hold, from the 16-byte fragments a lane keeps per
// block (the Q rows of its row tiles and one b x d key tile): sixteen waves
// (128 registers a lane) when they stay small, a single four-wave workgroup
// (the whole 512-register file) for the float32 shapes whose fragments
// alone would fill most of 256, eight waves otherwise.
template <int DT, int D, int B, int RT, int RG>
constexpr int score_wgs_per_cu() {
  constexpr int NV = D * Mma<DT>::kElemBytes / 64, F = (B / 16) * NV, RTW = RT / RG;
  constexpr int waves = score_waves<RG>();
  if (RG == 1 && B == 16 && (RTW + 1) * NV <= 8) return 16 / waves;
  if (RG == 1 && RTW * NV + F > 24) return 1;
  return kMaxWaves / waves;
}

// RG row groups: with two, waves 0-3 take the first half of the row tiles and
// waves 4-7 the second, both over all blocks, which halves the Q fragments a
// wave holds.
// FUSE: the workgroup also compacts its unit (compact_unit) after the
// selection.
template <int DT, int D, int B, int RT, int RG, bool FUSE>
__device__ __forceinline__ void score_unit(const ScoreParams& p) {
  constexpr int kWaves = score_waves<RG>();
  constexpr int kThreads = 64 * kWaves;
  constexpr int EB = Mma<DT>::kElemBytes;
  constexpr int NV = D * EB / 64;       // 16-byte fragments per lane per 16-token tile
  constexpr int NST = B / 16;           // 16-token sub-tiles per block
  constexpr int RTW = RT / RG;          // row tiles per wave
  constexpr int WPG = kWaves / RG;      // waves per row group
  constexpr int RPW = RTW * 16;         // rows per wave
  constexpr int ROWB = D * EB;          // bytes per key row
  constexpr int F = NST * NV;           // 16-byte fragments per lane per block
  // Shared tiles: with two row groups, the two waves of a pair (same blocks,
  // different rows) each load half of a block's fragments and swap the other
  // half through LDS, so every K byte is read from memory once per pass.
  // (Not for 16 fragments a lane, whose exchange buffers would not fit.)
  constexpr bool SH = RG == 2 && F <= 8;
  constexpr int FL = SH ? F / 2 : F;    // fragments a wave loads per block
  // K ring slots: as many block loads as fit the register budget, 2 to 4
  constexpr int kRingVgprs = RG == 2 ? ZP_SCORE_RING_VGPRS_2RG : ZP_SCORE_RING_VGPRS;
  constexpr int kPrefetch = kRingVgprs / (FL * 4) < 2   ? 2
                            : kRingVgprs / (FL * 4) > 4 ? 4
                                                        : kRingVgprs / (FL * 4);

  const size_t unit = (size_t)p.layer0 * p.R * p.H + blockIdx.x;  // over the whole call
  const int h = (int)(unit % p.H);
  const int lr = (int)(unit / p.H);
  const int l = lr / p.R, r = lr - l * p.R;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int rg = wave / WPG, wl = wave - rg * WPG;
  const char* kbase = static_cast<const char*>(p.layers[l - p.layer0].k);
  const char* qbase = static_cast<const char*>(p.layers[l - p.layer0].q);
  // the request's window rows: its own (r) or those of its query slot
  int qr = r;
  if (p.qslot) {
    qr = p.qslot[r];
    qr = (unsigned)qr < (unsigned)p.qslots ? qr : 0;
  }
  // this request's blocks and slots (the call's largest unless rows are ragged)
  const int n_src = unit_blocks(p.src, p.src_stride, r, p.n_src, p.n_max, p.ragged);
  const int T = n_src * B, C = T - p.w, E = T - p.K_keep;

  __shared__ __align__(16) float s_buf[lds_floats<RG>()];
  __shared__ float s_wst[kWaves][RPW][2];
  __shared__ float s_off[RT * 16];
  __shared__ float s_nrm[kWaves][B];
  __shared__ int s_scr[kWaves + 1];
  __shared__ __align__(16) SelectLds s_sel;
  __shared__ uint4 s_x[SH ? 2 : 1][SH ? WPG : 1][SH ? F : 1][64];  // [parity][pair][fragment][lane]
  // with shared tiles: per (row group, pair) the last exchange step whose
  // half that wave has written (steps numbered across both passes)
  __shared__ int s_pair[2][WPG];
  float* s_sc = s_buf;          // scores (with two row groups: group 0's partial importance)
  float* s_aux = s_buf + 4096;  // group 1's partial importance (two row groups only)
  float* s_rr = s_buf + 8192;   // redundancy (two row groups only)

  // query fragments: row = i*G + g is window position i of query head h*G+g
  uint4 qf[RTW][NV];
#pragma unroll
  for (int rt = 0; rt < RTW; rt++) {
    const int row = rg * RPW + rt * 16 + col;
    if (row < p.rows) {
      const int i = row / p.G, g = row - i * p.G;
      const char* ptr = qbase + ((size_t)(qr * p.w + i) * p.Hq + (size_t)h * p.G + g) * ROWB + grp * 16;
#pragma unroll
      for (int v = 0; v < NV; v++) qf[rt][v] = ld16(ptr + v * 64);
    } else {
#pragma unroll
      for (int v = 0; v < NV; v++) qf[rt][v] = make_uint4(0, 0, 0, 0);
    }
  }
  // last slot output row (rt, i) of this lane may attend to (causal window);
  // -1 for padding rows.  Only the last block needs it, so it is not kept.
  auto lim = [&](int rt, int i) {
    const int row = rg * RPW + rt * 16 + 4 * grp + i;
    return row < p.rows ? T - p.w + row / p.G : -1;
  };

  // this wave's blocks are wl + WPG*k; lane k holds the physical id of the k-th
  const int nbw = n_src > wl ? (n_src - wl + WPG - 1) / WPG : 0;
  // (a wave has at most 128 blocks: n_src <= 512 at four waves per row group)
  const int32_t* tab = p.src + (size_t)r * p.src_stride + wl;
  const int ids0 = lane < nbw ? tab[WPG * lane] : 0;
  const int ids1 = lane + 64 < nbw ? tab[WPG * (lane + 64)] : 0;
  const int row_off = col * ROWB + grp * 16;
  // K fragments of the wave's k-th block (k is clamped, so the loads stay
  // unconditional and the compiler can wait for each ring slot on its own).
  // Fragment f is sub-tile f / NV, 16-byte slice f % NV; with shared tiles a
  // wave loads fragments [rg*FL, rg*FL + FL).
  auto fetch = [&](int k, uint4 (&kd)[FL]) {
    const int kc = max(min(k, nbw - 1), 0);
    int pblk = kc < 64 ? __builtin_amdgcn_readlane(ids0, kc) : __builtin_amdgcn_readlane(ids1, kc - 64);
    pblk = (unsigned)pblk < (unsigned)p.num_blocks ? pblk : 0;  // never outside the pool
    const char* tile = kbase + ((size_t)pblk * p.H + h) * B * ROWB + row_off;
#pragma unroll
    for (int q = 0; q < FL; q++) {
      const int f = (SH ? rg * FL : 0) + q;
      kd[q] = ld16(tile + (f / NV) * 16 * ROWB + (f % NV) * 64);
    }
  };
  // Runs body(k, fragments) over the wave's blocks through a ring of PD
  // register buffers: slot s is refilled right after it is consumed, so
  // PD - 1 blocks stay in flight.  Pass 2 walks the blocks in reverse, so it
  // starts on those pass 1 read last (still in L2 / the memory-side cache).
  // With shared tiles only the two waves of a pair wait for each other: a
  // wave writes its half of the block, publishes the exchange step in
  // s_pair (release), and reads the partner's half once the partner has
  // published the same step (acquire).  Parity buffers alternate; a wave
  // overwrites one only after the partner has published the step after the
  // one that read it, so no half is overwritten before it is read.  Steps
  // are numbered from `base`, distinct per pass, so a pass never takes the
  // previous pass's counts for its own.  Both waves of a pair hold the same
  // blocks, so they run the same steps; the wait is bounded (2^16 sleeps)
  // so a wave can never spin forever.
  auto ring = [&](auto reverse, int base, auto body) {
    constexpr bool REV = decltype(reverse)::value;
    auto kof = [&](int it) { return REV ? nbw - 1 - it : it; };
    const int iters = SH ? (n_src + WPG - 1) / WPG : nbw;
    if (iters == 0) return;
    uint4 kb[kPrefetch][FL];
    // the prologue keeps slot order (the scheduler may not interleave the
    // fetches), so the wait before slot s counts the same loads on entry as
    // in the steady state
#pragma unroll
    for (int s = 0; s < kPrefetch; s++) {
      fetch(kof(s), kb[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int it0 = 0; it0 < iters; it0 += kPrefetch) {
#pragma unroll
      for (int s = 0; s < kPrefetch; s++) {
        const int it = it0 + s;
        if constexpr (SH) {
          if (it < iters) {
            const bool live = it < nbw;
            uint4* xb = &s_x[it & 1][wl][0][0];
            if (live) {
#pragma unroll
              for (int q = 0; q < FL; q++) xb[(rg * FL + q) * 64 + lane] = kb[s][q];
              // publish this half, then wait for the partner's (bounded)
              const int step = base + it + 1;
              __hip_atomic_store(&s_pair[rg][wl], step, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
              for (int spin = 0; spin < (1 << 16) &&
                   __hip_atomic_load(&s_pair[1 - rg][wl], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < step;
                   spin++)
                __builtin_amdgcn_s_sleep(1);
            }
            if (live) {
              uint4 kt[NST][NV];
#pragma unroll
              for (int f = 0; f < F; f++) {
                if (f / FL == rg)
                  kt[f / NV][f % NV] = kb[s][f % FL];
                else
                  kt[f / NV][f % NV] = xb[f * 64 + lane];
              }
              body(kof(it), kt);
            }
          }
        } else {
          if (it < nbw) {
            uint4 kt[NST][NV];
#pragma unroll
            for (int f = 0; f < F; f++) kt[f / NV][f % NV] = kb[s][f];
            body(kof(it), kt);
          }
        }
        fetch(kof(it + kPrefetch), kb[s]);
      }
    }
  };

  // phase boundaries on the device wall clock (debug only; thread 0)
  int64_t* const times = p.dbg_times ? p.dbg_times + unit * 5 : nullptr;
  auto stamp = [&](int k) {
    if (times && threadIdx.x == 0) times[k] = (int64_t)wall_clock64();
  };
  if constexpr (SH) {
    if (tid < 2 * WPG) (&s_pair[0][0])[tid] = 0;
    __syncthreads();
  }
  stamp(0);
  // ---------------------------------------------------------------- pass 1
  // Skipped when the caller supplies the normalisers of the window rows
  // (the log-sum-exp the decode steps of those rows computed over the same
  // slots): then K is read once.
  const float sl2 = p.scale_log2;
  const float* lse = p.layers[l - p.layer0].lse;
  if (lse != nullptr) {
    if (tid < RT * 16) {
      float o = 1.0e30f;  // padding rows: probability 0
      if (tid < p.rows) {
        const int i = tid / p.G, g = tid - i * p.G;
        const float v = lse[((size_t)qr * p.w + i) * p.Hq + (size_t)h * p.G + g];
        o = isfinite(v) ? v * 1.4426950408889634f : 1.0e30f;
      }
      s_off[tid] = o;
    }
  } else {
    float m[RTW][4], z[RTW][4];
#pragma unroll
    for (int rt = 0; rt < RTW; rt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        m[rt][i] = kInitMax;
        z[rt][i] = 0.f;
      }
    ring(BoolC<false>{}, 0, [&](int k, const uint4 (&kt)[NST][NV]) {
      const int n = wl + WPG * k;
      const bool last = n == n_src - 1;  // only the last block meets the causal limit
#pragma unroll
      for (int st = 0; st < NST; st++) {
        const int j = n * B + st * 16 + col;
        f32x4_t acc[RTW];
#pragma unroll
        for (int rt = 0; rt < RTW; rt++) {
          acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int v = 0; v < NV; v++) acc[rt] = Mma<DT>::step(qf[rt][v], kt[st][v], acc[rt]);
        }
        // 2^(x - m) for every logit; a term above 2^kLazy (or the causal
        // block) sends the lane through the rescaling update instead
        float e[RTW][4];
        bool slow = last;
#pragma unroll
        for (int rt = 0; rt < RTW; rt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            e[rt][i] = fast_exp2(fmaf(acc[rt][i], sl2, -m[rt][i]));
            slow |= e[rt][i] > kLazyTerm;
          }
        if (slow) {
#pragma unroll
          for (int rt = 0; rt < RTW; rt++)
#pragma unroll
            for (int i = 0; i < 4; i++)
              lazy_update(m[rt][i], z[rt][i], j <= lim(rt, i) ? acc[rt][i] * sl2 : kMasked);
        } else {
#pragma unroll
          for (int rt = 0; rt < RTW; rt++)
#pragma unroll
            for (int i = 0; i < 4; i++) z[rt][i] += e[rt][i];
        }
      }
    });
    // merge the 16 columns of every row (DPP inside 16-lane rows)
#pragma unroll
    for (int rt = 0; rt < RTW; rt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        merge_dpp<0xB1>(m[rt][i], z[rt][i]);   // quad_perm [1,0,3,2]
        merge_dpp<0x4E>(m[rt][i], z[rt][i]);   // quad_perm [2,3,0,1]
        merge_dpp<0x141>(m[rt][i], z[rt][i]);  // row_half_mirror
        merge_dpp<0x140>(m[rt][i], z[rt][i]);  // row_mirror
      }
    if (col == 0) {
#pragma unroll
      for (int rt = 0; rt < RTW; rt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          s_wst[wave][rt * 16 + 4 * grp + i][0] = m[rt][i];
          s_wst[wave][rt * 16 + 4 * grp + i][1] = z[rt][i];
        }
    }
    __syncthreads();
    if (tid < RT * 16) {
      const int g = tid / RPW, row = tid - g * RPW;
      float M = kInitMax, Z = 0.f;
      for (int w = g * WPG; w < (g + 1) * WPG; w++) merge_stat(M, Z, s_wst[w][row][0], s_wst[w][row][1]);
      // probability of a logit x (log2 units) in this row: 2^(x - offset)
      s_off[tid] = Z > 0.f ? M + fast_log2(Z) : 1.0e30f;
    }
  }
  __syncthreads();
  float off[RTW][4];
#pragma unroll
  for (int rt = 0; rt < RTW; rt++)
#pragma unroll
    for (int i = 0; i < 4; i++) off[rt][i] = s_off[rg * RPW + rt * 16 + 4 * grp + i];

  stamp(1);
  // ---------------------------------------------------------------- pass 2
  const float inv_rows = 1.0f / (float)p.rows;
  const float inv_bm1 = 1.0f / (float)(B - 1);
  // column sums of the probabilities of sub-tile st (causal mask: last block only)
  auto prob_sum = [&](auto lastc, int j, const uint4 (&kf)[NV]) {
    constexpr bool LAST = decltype(lastc)::value;
    float cs = 0.f;
#pragma unroll
    for (int rt = 0; rt < RTW; rt++) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < NV; v++) acc = Mma<DT>::step(qf[rt][v], kf[v], acc);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float pr = fast_exp2(fmaf(acc[i], sl2, -off[rt][i]));
        cs += (!LAST || j <= lim(rt, i)) ? pr : 0.f;
      }
    }
    return sum_rows(cs);
  };
  ring(BoolC<kReversePass2>{}, 1 << 16, [&](int k, const uint4 (&kt)[NST][NV]) {
    const int n = wl + WPG * k;
    const bool last = n == n_src - 1;
    float A[NST];
#pragma unroll
    for (int st = 0; st < NST; st++) {
      const int j = n * B + st * 16 + col;
      A[st] = last ? prob_sum(BoolC<true>{}, j, kt[st]) : prob_sum(BoolC<false>{}, j, kt[st]);
    }
    if (RG == 2 && grp == 0) {
      float* dst = rg == 0 ? s_sc : s_aux;
#pragma unroll
      for (int st = 0; st < NST; st++) dst[n * B + st * 16 + col] = A[st];
    }
    // the two row groups see the same blocks: they take turns on the Gram
    // work, whole blocks each (splitting a block's Gram between the pair
    // costs more: both waves then need the diagonal tiles for the norms)
    if (RG == 1 || (k & 1) == rg) {
      // redundancy: column sums of the in-block cosine matrix, diagonal
      // excluded.  gm[s1][s2] holds the dot products of keys 16*s1 + 4*grp + i
      // (rows) with keys 16*s2 + col; the diagonal tiles give the squared
      // norms, and the inverse norms of a lane's rows come through LDS.
      f32x4_t gm[NST][NST];
#pragma unroll
      for (int s1 = 0; s1 < NST; s1++)
#pragma unroll
        for (int s2 = 0; s2 < NST; s2++) {
          gm[s1][s2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int v = 0; v < NV; v++) gm[s1][s2] = Mma<DT>::step(kt[s1][v], kt[s2][v], gm[s1][s2]);
        }
      float nrm[NST];
#pragma unroll
      for (int st = 0; st < NST; st++) {
        const f32x4_t g = gm[st][st];
        const int e = col & 3;
        float dg = e == 0 ? g[0] : e == 1 ? g[1] : e == 2 ? g[2] : g[3];
        dg = (col >> 2) == grp ? dg : 0.f;  // lane (col/4, col) holds key col's diagonal entry
        nrm[st] = sum_rows(dg);
      }
      if (grp == 0) {
#pragma unroll
        for (int st = 0; st < NST; st++) s_nrm[wave][st * 16 + col] = nrm[st];
      }
      __builtin_amdgcn_wave_barrier();
      float ra[NST][4];
#pragma unroll
      for (int s1 = 0; s1 < NST; s1++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float na = s_nrm[wave][s1 * 16 + 4 * grp + i];
          ra[s1][i] = na > 0.f ? rsqrtf(na) : 0.f;
        }
      __builtin_amdgcn_wave_barrier();
      float Rd[NST];
#pragma unroll
      for (int s2 = 0; s2 < NST; s2++) {
        // the column's inverse norm is common to all its terms (every lane
        // of the column holds the same one), so it multiplies the sum
        float cs = 0.f;
        const float rc = nrm[s2] > 0.f ? rsqrtf(nrm[s2]) : 0.f;
#pragma unroll
        for (int s1 = 0; s1 < NST; s1++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const bool diag = (s1 == s2) && (4 * grp + i == col);
            cs += diag ? 0.f : gm[s1][s2][i] * ra[s1][i];
          }
        Rd[s2] = sum_rows(cs * rc) * inv_bm1;
      }
      if (grp == 0) {
#pragma unroll
        for (int st = 0; st < NST; st++) {
          const int j = n * B + st * 16 + col;
          if (RG == 1) {
            const float a = A[st] * inv_rows;
            const float s = a * (1.0f - Rd[st]);
            s_sc[j] = s;
            const size_t o = unit * p.T + j;
            if (p.dbg_importance) p.dbg_importance[o] = a;
            if (p.dbg_redundancy) p.dbg_redundancy[o] = Rd[st];
            if (p.dbg_score && j < C) p.dbg_score[o] = s;
          } else {
            s_rr[j] = Rd[st];
          }
        }
      }
    }
  });
  __syncthreads();
  if (RG == 2) {
    for (int j = tid; j < T; j += kThreads) {
      const float a = (s_sc[j] + s_aux[j]) * inv_rows;
      const float s = a * (1.0f - s_rr[j]);
      const size_t o = unit * p.T + j;
      if (p.dbg_importance) p.dbg_importance[o] = a;
      if (p.dbg_redundancy) p.dbg_redundancy[o] = s_rr[j];
      if (p.dbg_score && j < C) p.dbg_score[o] = s;
      s_sc[j] = s;
    }
    __syncthreads();
  }

  stamp(2);
  // ---------------------------------------------------------------- select
  const int per = (T + kThreads - 1) / kThreads;
  int* s_f = FUSE ? reinterpret_cast<int*>(s_buf) : nullptr;  // the scores are in registers by then
  if (per <= 8) select_evicted<8, kWaves>(s_sc, s_sel, s_scr, p, unit, s_f, T, C, E);
  else if (per <= 16) select_evicted<16, kWaves>(s_sc, s_sel, s_scr, p, unit, s_f, T, C, E);
  else select_evicted<32, kWaves>(s_sc, s_sel, s_scr, p, unit, s_f, T, C, E);
  stamp(3);
  if constexpr (FUSE) {
    // rows a thread moves per tile: half as many where sixteen waves share a
    // CU (128 registers a lane), so the tile buffers fit beside the scoring's
    constexpr int kU = score_wgs_per_cu<DT, D, B, RT, RG>() * kWaves > kMaxWaves ? kFusedUnroll / 2
                                                                                : kFusedUnroll;
    __shared__ int s_first;
    if (p.k_cached)  // uniform: one tile loop or the other, each straight-line
      compact_unit<ROWB / 16, B, kThreads, kU, true>(p, s_buf, &s_first, l, r, h, n_src, E);
    else
      compact_unit<ROWB / 16, B, kThreads, kU, false>(p, s_buf, &s_first, l, r, h, n_src, E);
  }
  if (times) {
    __syncthreads();  // every wave done (uniform: the pointer is a kernel argument)
    stamp(4);
  }
}

template <int DT, int D, int B, int RT, int RG>
__global__ __launch_bounds__(64 * score_waves<RG>(), (score_wgs_per_cu<DT, D, B, RT, RG>())) void k_score_select(ScoreParams p) {
  score_unit<DT, D, B, RT, RG, false>(p);
}

template <int DT, int D, int B, int RT, int RG>
__global__ __launch_bounds__(64 * score_waves<RG>(), (score_wgs_per_cu<DT, D, B, RT, RG>())) void k_score_compact(ScoreParams p) {
  score_unit<DT, D, B, RT, RG, true>(p);
}

// Workgroups of one instantiation that a compute unit holds at once (from
// the compiled kernel's registers, LDS and launch bounds).
template <int DT, int D, int B, int RT, int RG>
hipError_t resident_rt(bool fused, int* per_cu) {
  const auto fn = fused ? reinterpret_cast<const void*>(&k_score_compact<DT, D, B, RT, RG>)
                        : reinterpret_cast<const void*>(&k_score_select<DT, D, B, RT, RG>);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, fn, 64 * score_waves<RG>(), 0);
}

template <int DT, int D, int B, int RT, int RG>
hipError_t launch_rt(const ScoreParams& p, int units, hipStream_t s) {
  const dim3 grid(units), block(64 * score_waves<RG>());
  if (p.dst) {
    prof_begin(ZP_PHASE_SCORE_COMPACT, s);
    hipLaunchKernelGGL((k_score_compact<DT, D, B, RT, RG>), grid, block, 0, s, p);
    prof_end(ZP_PHASE_SCORE_COMPACT, s);
  } else {
    prof_begin(ZP_PHASE_SCORE, s);
    hipLaunchKernelGGL((k_score_select<DT, D, B, RT, RG>), grid, block, 0, s, p);
    prof_end(ZP_PHASE_SCORE, s);
  }
  return hipGetLastError();
}

template <int DT, int D, int B>
hipError_t resident_b(bool fused, int row_tiles, int T, int* per_cu) {
  switch (row_tiles) {
    case 1: return resident_rt<DT, D, B, 1, 1>(fused, per_cu);
    case 2: return resident_rt<DT, D, B, 2, 1>(fused, per_cu);
    case 4: return resident_rt<DT, D, B, 4, 1>(fused, per_cu);
    case 8: return score_two_groups(8, T) ? resident_rt<DT, D, B, 8, 2>(fused, per_cu)
                                          : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template <int DT, int D, int B>
hipError_t launch_b(const ScoreParams& p, int row_tiles, int units, hipStream_t s) {
  const bool two_groups = score_two_groups(row_tiles, p.T);
  switch (row_tiles) {
    case 1: return launch_rt<DT, D, B, 1, 1>(p, units, s);
    case 2: return launch_rt<DT, D, B, 2, 1>(p, units, s);
    case 4: return launch_rt<DT, D, B, 4, 1>(p, units, s);
    case 8: return two_groups ? launch_rt<DT, D, B, 8, 2>(p, units, s) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template <int DT, int D>
hipError_t launch_d(const ScoreParams& p, int block_size, int row_tiles, int units, hipStream_t s) {
  if (block_size == 16) return launch_b<DT, D, 16>(p, row_tiles, units, s);
  if (block_size == 32) return launch_b<DT, D, 32>(p, row_tiles, units, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const ScoreParams& p, int head_dim, int block_size, int row_tiles, int units,
                     hipStream_t s) {
  if (head_dim == 64) return launch_d<DT, 64>(p, block_size, row_tiles, units, s);
  if (head_dim == 128) return launch_d<DT, 128>(p, block_size, row_tiles, units, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t resident_dt(bool fused, int head_dim, int block_size, int row_tiles, int T, int* per_cu) {
  if (head_dim == 64 && block_size == 16) return resident_b<DT, 64, 16>(fused, row_tiles, T, per_cu);
  if (head_dim == 64 && block_size == 32) return resident_b<DT, 64, 32>(fused, row_tiles, T, per_cu);
  if (head_dim == 128 && block_size == 16) return resident_b<DT, 128, 16>(fused, row_tiles, T, per_cu);
  if (head_dim == 128 && block_size == 32) return resident_b<DT, 128, 32>(fused, row_tiles, T, per_cu);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t score_resident_per_cu(int dtype, int head_dim, int block_size, int rows, int T,
                                 bool fused, int* per_cu) {
  if (!score_fits(rows, T)) return hipErrorInvalidValue;
  const int rt = score_row_tiles(rows);
  if (dtype == ZP_BF16) return resident_dt<ZP_BF16>(fused, head_dim, block_size, rt, T, per_cu);
  if (dtype == ZP_F32) return resident_dt<ZP_F32>(fused, head_dim, block_size, rt, T, per_cu);
  return hipErrorInvalidValue;
}

hipError_t launch_score(const ScoreParams& p, int dtype, int head_dim, int block_size, int units,
                        hipStream_t s) {
  if (units <= 0) return hipSuccess;
  if (!score_fits(p.rows, p.T)) return hipErrorInvalidValue;
  // the fused compaction's LDS lists: E evicted slots, n_src <= 512 blocks
  if (p.dst && (p.E < 0 || p.E > kMaxEvicted || p.n_src > kMaxScoreSlots / 16 || p.n_max < 2 ||
                p.n_max > p.n_src || p.K_keep != (p.n_max - 1) * block_size))
    return hipErrorInvalidValue;
  const int rt = score_row_tiles(p.rows);
  if (dtype == ZP_BF16) return launch_dt<ZP_BF16>(p, head_dim, block_size, rt, units, s);
  if (dtype == ZP_F32) return launch_dt<ZP_F32>(p, head_dim, block_size, rt, units, s);
  return hipErrorInvalidValue;
}

}  // namespace zp
