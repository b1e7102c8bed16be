/*
 * zp_oracle.c -- plain, slow CPU oracle for Compressed PagedAttention
 * (the Zipage compression pass over a paged KV cache, and paged decode).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  The HIP library
 * never links, includes or calls it, and it includes nothing from there.
 *
 * Arithmetic: every stored value is widened exactly (bfloat16 -> double,
 * float -> double) and all scores, softmaxes and dot products are computed
 * in double.  No blocking, no fusion, no reordering beyond the definitions
 * below.  Parallelism (OpenMP) is only over independent (request, head)
 * units and never changes a result.
 *
 * Sources (the Zipage summaries at gist.science/nl/paper/2603.08743, page 1,
 * "Technische samenvatting"; gist.science/ko/paper/2603.08743, page 2,
 * "기술 요약"; and the paged-KV-cache guide at upskillscore.com, page 3):
 *   - trigger, relocation into the first N_max-1 blocks, reserved last
 *     block, release of surplus blocks: page 1 Methodologie item 1,
 *     page 2 section 2.A;
 *   - per-layer, per-head token-wise eviction: page 2 section 2.A;
 *   - observation window of the most recent w tokens of the last block,
 *     window always kept: page 2 section 2.A;
 *   - Lightning Redundancy Score, similarity only between tokens of the same
 *     block, O(N b^2): page 1 Methodologie item 5, page 2 section 2.E;
 *   - compression into newly allocated target blocks when blocks are shared,
 *     reference counts kept: page 1 Methodologie item 3, page 2 section 2.C;
 *   - block tables, reference counts, copy-on-write that allocates and
 *     decrements: page 3 "How it works".
 * Readings where the pages are silent (all stated again in the design notes):
 *   - importance of slot j = mean over the G*w (query head, window row)
 *     pairs of the causal softmax probability of j;
 *   - redundancy of slot j = mean cosine similarity with the other b-1 keys
 *     of its block (0 for a zero-norm key);
 *   - combined score s = A * (1 - R); ties: lower logical slot kept;
 *   - survivors = K_sel best candidates plus the w window slots, in
 *     ascending slot order.
 *
 * Parity note: every function here is pinned by CPU tests against brute
 * force, closed forms, library routines or invariants, the three readings
 * above included (combination s = A(1-R), mean over the group, mean
 * cosine: a hand-worked example with exact rational values, SciPy's softmax,
 * scikit-learn's cosine).  What no test can pin is that the pages meant
 * these readings: they print no number for them, so the choices themselves
 * are fixed here and in the library header, not confirmed.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ZPO_OK 0
#define ZPO_INVALID 1
#define ZPO_NO_BLOCKS 2

/* Exact widening of one stored element (bf16 bit pattern or float32). */
static double widen(const void* base, size_t idx, int is_bf16) {
  if (is_bf16) {
    uint32_t u = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

/* Address (in elements) of row (block, head, offset) in a [nb][H][b][d] pool. */
static size_t row_index(int32_t block, int h, int off, int H, int b, int d) {
  return (((size_t)block * (size_t)H + (size_t)h) * (size_t)b + (size_t)off) * (size_t)d;
}

int zpo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------
 * Planning (trigger already decided by the caller: every listed request
 * holds n_src >= n_max full blocks; n_src > n_max is a cache that grew past
 * the cap, e.g. a long prompt, whose surplus blocks are released).
 *
 * Reference counts are read at the start of the call.  For each request,
 * in order, and each logical block n < n_max-1: a block referenced only by
 * this request is compacted in place; a shared one gets a new target block
 * (the smallest free id) and this request drops its reference to the
 * shared source.  Logical block n_max-1 is kept as the reserved block if
 * private, otherwise replaced by a fresh block.  Blocks n_max..n_src-1 are
 * surplus: the request drops its reference to each.  Blocks whose count
 * reaches zero are reported as freed.  Nothing is changed when the inputs
 * are invalid or when too few blocks are free.
 *
 * tables: [R][n_src] in; out: the n_max new ids, then -1 for the surplus.
 * src_out: [R][n_src] (the old table).  dst_out: [R][n_max-1] (compaction
 * targets).  freed_out: capacity R*n_src.
 *
 * first_evict (NULL, or [R]): the request's lowest evicted slot over all
 * layers and heads.  A shared block n < n_max-1 whose slots all lie below it
 * is left as it is in every layer and head by the compaction, so it stays in
 * the table, still shared (no new target, counts unchanged).
 *
 * n_blocks (NULL, or [R]): requests past the cap by different amounts in one
 * call; request r holds the first n_blocks[r] entries of its row (between
 * n_max and n_src) and the rest of the row is -1.  Everything above then
 * reads n_blocks[r] for n_src, request by request, in the same order.
 * --------------------------------------------------------------------- */
int zpo_plan(int32_t pool_size, int32_t* rc, int32_t R, int32_t n_src, int32_t n_max,
             int32_t* tables, int32_t* src_out, int32_t* dst_out, int32_t* freed_out,
             int32_t* n_freed_out, const int32_t* first_evict, int32_t b,
             const int32_t* n_blocks) {
  if (pool_size <= 0 || R < 0 || n_max < 2 || n_src < n_max) return ZPO_INVALID;
  /* n_blocks (optional): request r holds the first n_blocks[r] entries of
   * its row, n_max <= n_blocks[r] <= n_src; the rest of the row is -1 */
  if (n_blocks)
    for (int32_t r = 0; r < R; r++) {
      if (n_blocks[r] < n_max || n_blocks[r] > n_src) return ZPO_INVALID;
      for (int32_t n = n_blocks[r]; n < n_src; n++)
        if (tables[(size_t)r * n_src + n] != -1) return ZPO_INVALID;
    }
  int32_t* seen = (int32_t*)calloc((size_t)pool_size, sizeof(int32_t));
  int32_t* rc0 = (int32_t*)malloc((size_t)pool_size * sizeof(int32_t));
  if (!seen || !rc0) { free(seen); free(rc0); return ZPO_INVALID; }
  memcpy(rc0, rc, (size_t)pool_size * sizeof(int32_t));
  int bad = 0;
  for (int32_t r = 0; r < R && !bad; r++) {
    const int32_t nr = n_blocks ? n_blocks[r] : n_src;
    for (int32_t n = 0; n < nr && !bad; n++) {
      int32_t id = tables[(size_t)r * n_src + n];
      if (id < 0 || id >= pool_size || rc0[id] < 1) { bad = 1; break; }
      for (int32_t m = 0; m < n; m++)
        if (tables[(size_t)r * n_src + m] == id) { bad = 1; break; }
      seen[id] += 1;
      if (seen[id] > rc0[id]) bad = 1;
    }
  }
  if (bad) { free(seen); free(rc0); return ZPO_INVALID; }
  int64_t need = 0, nfree = 0;
  for (int32_t r = 0; r < R; r++)
    for (int32_t n = 0; n < n_max; n++) {
      const int stays = first_evict && n < n_max - 1 && (int64_t)(n + 1) * b <= first_evict[r];
      if (rc0[tables[(size_t)r * n_src + n]] > 1 && !stays) need++;
    }
  for (int32_t i = 0; i < pool_size; i++)
    if (rc0[i] == 0) nfree++;
  if (need > nfree) { free(seen); free(rc0); return ZPO_NO_BLOCKS; }

  int32_t next_free = 0; /* scan pointer over ids that were free at the start */
  int32_t nfreed = 0;
  for (int32_t r = 0; r < R; r++) {
    int32_t* row = tables + (size_t)r * n_src;
    const int32_t nr = n_blocks ? n_blocks[r] : n_src;
    for (int32_t n = 0; n < n_src; n++) src_out[(size_t)r * n_src + n] = row[n];
    for (int32_t n = 0; n < nr; n++) {
      int32_t s = row[n];
      if (n >= n_max) { /* surplus: released */
        rc[s] -= 1;
        if (rc[s] == 0) freed_out[nfreed++] = s;
        row[n] = -1;
        continue;
      }
      int32_t target = s;
      const int stays = first_evict && n < n_max - 1 && (int64_t)(n + 1) * b <= first_evict[r];
      if (rc0[s] > 1 && !stays) {
        while (rc0[next_free] != 0) next_free++;
        target = next_free++;
        rc[target] = 1;
        rc[s] -= 1;
        if (rc[s] == 0) freed_out[nfreed++] = s;
      }
      if (n < n_max - 1) dst_out[(size_t)r * (n_max - 1) + n] = target;
      row[n] = target;
    }
  }
  *n_freed_out = nfreed;
  free(seen);
  free(rc0);
  return ZPO_OK;
}

/* ---------------------------------------------------------------------
 * Scores for one layer.  Per request r and KV head h (G = Hq/H query heads
 * per KV head), with T = n_src*b cached slots read through the block table:
 *   importance A[j] = 1/(G w) * sum over g < G, i < w with p_i >= j of
 *       softmax over slots 0..p_i of x_{g,i}, where p_i = T-w+i and
 *       x_{g,i}[j] = q_{i, hG+g} . k_j / sqrt(d)   (causal window queries);
 *   redundancy R[j] = 1/(b-1) * sum over the other slots c of j's block of
 *       cos(k_j, k_c), with cos = 0 when either norm is 0;
 *   s[j] = A[j] * (1 - R[j]) for the candidates j < T-w; NaN elsewhere.
 * Outputs are [R][H][T] doubles.
 * --------------------------------------------------------------------- */
void zpo_scores(int32_t H, int32_t Hq, int32_t d, int32_t b, int32_t is_bf16, int32_t n_src,
                int32_t w, int32_t R, const void* kpool, const void* window_q,
                const int32_t* src, double* A_out, double* R_out, double* s_out) {
  const int32_t G = Hq / H;
  const int32_t T = n_src * b;
  const int32_t C = T - w;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < (int64_t)R * H; unit++) {
    const int32_t r = (int32_t)(unit / H), h = (int32_t)(unit % H);
    /* logical keys of this (request, head) */
    double* K = (double*)malloc((size_t)T * d * sizeof(double));
    double* P = (double*)calloc((size_t)T, sizeof(double));
    double* x = (double*)malloc((size_t)T * sizeof(double));
    double* q = (double*)malloc((size_t)d * sizeof(double));
    double* nrm = (double*)malloc((size_t)T * sizeof(double));
    for (int32_t j = 0; j < T; j++) {
      int32_t blk = src[(size_t)r * n_src + j / b];
      size_t base = row_index(blk, h, j % b, H, b, d);
      for (int32_t e = 0; e < d; e++) K[(size_t)j * d + e] = widen(kpool, base + e, is_bf16);
    }
    /* importance */
    for (int32_t g = 0; g < G; g++) {
      for (int32_t i = 0; i < w; i++) {
        const int32_t p = T - w + i;
        size_t qbase = (((size_t)r * w + i) * Hq + (size_t)h * G + g) * d;
        for (int32_t e = 0; e < d; e++) q[e] = widen(window_q, qbase + e, is_bf16);
        double m = -INFINITY;
        for (int32_t j = 0; j <= p; j++) {
          double dot = 0.0;
          for (int32_t e = 0; e < d; e++) dot += q[e] * K[(size_t)j * d + e];
          x[j] = dot * inv_sqrt_d;
          if (x[j] > m) m = x[j];
        }
        double Z = 0.0;
        for (int32_t j = 0; j <= p; j++) Z += exp(x[j] - m);
        for (int32_t j = 0; j <= p; j++) P[j] += exp(x[j] - m) / Z;
      }
    }
    double* Ao = A_out + ((size_t)r * H + h) * T;
    double* Ro = R_out + ((size_t)r * H + h) * T;
    double* so = s_out + ((size_t)r * H + h) * T;
    for (int32_t j = 0; j < T; j++) Ao[j] = P[j] / (double)(G * w);
    /* Lightning Redundancy Score: cosine only inside each block */
    for (int32_t j = 0; j < T; j++) {
      double ss = 0.0;
      for (int32_t e = 0; e < d; e++) ss += K[(size_t)j * d + e] * K[(size_t)j * d + e];
      nrm[j] = sqrt(ss);
    }
    for (int32_t n = 0; n < n_src; n++) {
      for (int32_t a = 0; a < b; a++) {
        const int32_t ja = n * b + a;
        double acc = 0.0;
        for (int32_t c = 0; c < b; c++) {
          const int32_t jc = n * b + c;
          if (c == a) continue;
          if (nrm[ja] == 0.0 || nrm[jc] == 0.0) continue;
          double dot = 0.0;
          for (int32_t e = 0; e < d; e++) dot += K[(size_t)ja * d + e] * K[(size_t)jc * d + e];
          acc += dot / (nrm[ja] * nrm[jc]);
        }
        Ro[ja] = acc / (double)(b - 1);
      }
    }
    for (int32_t j = 0; j < T; j++) so[j] = (j < C) ? Ao[j] * (1.0 - Ro[j]) : NAN;
    free(K); free(P); free(x); free(q); free(nrm);
  }
}

/* ---------------------------------------------------------------------
 * Selection.  Per (request, head): sort all candidates j < C = T-w by
 * (s descending, j ascending), keep the first k_sel, add the window slots
 * C..T-1, and list the survivors in ascending slot order.
 * s: [units][T] doubles; kept: [units][k_sel + w].
 * --------------------------------------------------------------------- */
typedef struct { double s; int32_t j; } zpo_cand;

static int cand_order(const void* pa, const void* pb) {
  const zpo_cand* a = (const zpo_cand*)pa;
  const zpo_cand* b = (const zpo_cand*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

void zpo_select(int64_t units, int32_t T, int32_t w, int32_t k_sel, const double* s,
                int32_t* kept) {
  const int32_t C = T - w;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t u = 0; u < units; u++) {
    zpo_cand* c = (zpo_cand*)malloc((size_t)C * sizeof(zpo_cand));
    unsigned char* keep = (unsigned char*)calloc((size_t)T, 1);
    for (int32_t j = 0; j < C; j++) { c[j].s = s[(size_t)u * T + j]; c[j].j = j; }
    qsort(c, (size_t)C, sizeof(zpo_cand), cand_order);
    for (int32_t k = 0; k < k_sel; k++) keep[c[k].j] = 1;
    for (int32_t j = C; j < T; j++) keep[j] = 1;
    int32_t r = 0;
    for (int32_t j = 0; j < T; j++)
      if (keep[j]) kept[(size_t)u * (k_sel + w) + r++] = j;
    free(c);
    free(keep);
  }
}

/* ---------------------------------------------------------------------
 * Order-preserving compaction of one pool (K or V of one layer), out of
 * place: pool_out starts as a copy of pool_in, then for every request and
 * head, new logical slot r (in the dst blocks) receives old logical slot
 * kept[r] (read through the src table from pool_in).
 * src: [R][n_src], dst: [R][n_max-1], kept: [R][H][k_keep].
 * --------------------------------------------------------------------- */
void zpo_compact(int64_t pool_elems, int32_t H, int32_t d, int32_t b, int32_t elem_bytes,
                 int32_t n_src, int32_t n_max, int32_t R, int32_t k_keep, const void* pool_in,
                 void* pool_out, const int32_t* src, const int32_t* dst, const int32_t* kept) {
  memcpy(pool_out, pool_in, (size_t)pool_elems * (size_t)elem_bytes);
  const size_t row_bytes = (size_t)d * (size_t)elem_bytes;
  for (int32_t r = 0; r < R; r++) {
    for (int32_t h = 0; h < H; h++) {
      const int32_t* kp = kept + ((size_t)r * H + h) * k_keep;
      for (int32_t slot = 0; slot < k_keep; slot++) {
        int32_t j = kp[slot];
        int32_t sblk = src[(size_t)r * n_src + j / b];
        int32_t dblk = dst[(size_t)r * (n_max - 1) + slot / b];
        const char* from = (const char*)pool_in + row_index(sblk, h, j % b, H, b, d) * elem_bytes;
        char* to = (char*)pool_out + row_index(dblk, h, slot % b, H, b, d) * elem_bytes;
        memcpy(to, from, row_bytes);
      }
    }
  }
}

/* ---------------------------------------------------------------------
 * Append one token per request: k_new/v_new [R][H][d] written to physical
 * slot slot_mapping[r] = block*b + offset of every head.
 * --------------------------------------------------------------------- */
void zpo_append(int32_t H, int32_t d, int32_t b, int32_t elem_bytes, int32_t R, void* kpool,
                void* vpool, const void* k_new, const void* v_new, const int32_t* slot_mapping) {
  const size_t row_bytes = (size_t)d * (size_t)elem_bytes;
  for (int32_t r = 0; r < R; r++) {
    int32_t blk = slot_mapping[r] / b, off = slot_mapping[r] % b;
    for (int32_t h = 0; h < H; h++) {
      size_t to = row_index(blk, h, off, H, b, d) * elem_bytes;
      size_t from = ((size_t)r * H + h) * row_bytes;
      memcpy((char*)kpool + to, (const char*)k_new + from, row_bytes);
      memcpy((char*)vpool + to, (const char*)v_new + from, row_bytes);
    }
  }
}

/* ---------------------------------------------------------------------
 * Paged decode attention, dense: for request r and query head hq (KV head
 * hq/G), out = sum over j < seq_len of softmax_j(scale * q . k_j) * v_j,
 * with slot j at block tables[r][j/b], offset j%b.  out: [R][Hq][d] doubles.
 * --------------------------------------------------------------------- */
void zpo_decode(int32_t H, int32_t Hq, int32_t d, int32_t b, int32_t is_bf16, int32_t R,
                const void* kpool, const void* vpool, const void* q, const int32_t* tables,
                int32_t max_blocks, const int32_t* seq_lens, double scale, double* out) {
  const int32_t G = Hq / H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < (int64_t)R * Hq; unit++) {
    const int32_t r = (int32_t)(unit / Hq), hq = (int32_t)(unit % Hq), h = hq / G;
    const int32_t n = seq_lens[r];
    double* x = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double* qv = (double*)malloc((size_t)d * sizeof(double));
    double* o = out + ((size_t)r * Hq + hq) * d;
    for (int32_t e = 0; e < d; e++) qv[e] = widen(q, ((size_t)r * Hq + hq) * d + e, is_bf16);
    double m = -INFINITY;
    for (int32_t j = 0; j < n; j++) {
      int32_t blk = tables[(size_t)r * max_blocks + j / b];
      size_t base = row_index(blk, h, j % b, H, b, d);
      double dot = 0.0;
      for (int32_t e = 0; e < d; e++) dot += qv[e] * widen(kpool, base + e, is_bf16);
      x[j] = scale * dot;
      if (x[j] > m) m = x[j];
    }
    double Z = 0.0;
    for (int32_t j = 0; j < n; j++) Z += exp(x[j] - m);
    for (int32_t e = 0; e < d; e++) o[e] = 0.0;
    for (int32_t j = 0; j < n; j++) {
      int32_t blk = tables[(size_t)r * max_blocks + j / b];
      size_t base = row_index(blk, h, j % b, H, b, d);
      double p = exp(x[j] - m) / Z;
      for (int32_t e = 0; e < d; e++) o[e] += p * widen(vpool, base + e, is_bf16);
    }
    free(x);
    free(qv);
  }
}

/* ---------------------------------------------------------------------
 * Log-sum-exp of the decode logits: for request r and query head hq (KV
 * head hq/G), lse = log sum over j < seq_len of exp(scale * q . k_j), with
 * slot j at block tables[r][j/b], offset j%b; -inf for an empty request.
 * This is the normaliser of the softmax in zpo_decode; the same quantity
 * for a window query over slots 0..C+i is the normaliser of that window
 * row's importance softmax.  lse: [R][Hq] doubles.
 * --------------------------------------------------------------------- */
void zpo_decode_lse(int32_t H, int32_t Hq, int32_t d, int32_t b, int32_t is_bf16, int32_t R,
                    const void* kpool, const void* q, const int32_t* tables, int32_t max_blocks,
                    const int32_t* seq_lens, double scale, double* lse) {
  const int32_t G = Hq / H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < (int64_t)R * Hq; unit++) {
    const int32_t r = (int32_t)(unit / Hq), hq = (int32_t)(unit % Hq), h = hq / G;
    const int32_t n = seq_lens[r];
    double* x = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double m = -INFINITY;
    for (int32_t j = 0; j < n; j++) {
      int32_t blk = tables[(size_t)r * max_blocks + j / b];
      size_t base = row_index(blk, h, j % b, H, b, d);
      double dot = 0.0;
      for (int32_t e = 0; e < d; e++)
        dot += widen(q, ((size_t)r * Hq + hq) * d + e, is_bf16) * widen(kpool, base + e, is_bf16);
      x[j] = scale * dot;
      if (x[j] > m) m = x[j];
    }
    double Z = 0.0;
    for (int32_t j = 0; j < n; j++) Z += exp(x[j] - m);
    lse[(size_t)r * Hq + hq] = n > 0 ? m + log(Z) : -INFINITY;
    free(x);
  }
}

/* ---------------------------------------------------------------------
 * All-pairs redundancy (the pairwise computation the Lightning Redundancy
 * Score replaces: O(N^2 b^2) pairs instead of O(N b^2); nl page
 * Methodologie item 5, ko page section 2.E).  Same reduction as the LRS,
 * over the whole sequence instead of the block: for request r, head h and
 * each of the T = n_blocks*b slots j,
 *   R_all[j] = 1/(T-1) * sum over c != j of cos(k_j, k_c)   (0 for a zero norm).
 * out: [R][H][T] doubles.
 * --------------------------------------------------------------------- */
void zpo_redundancy_all(int32_t H, int32_t d, int32_t b, int32_t is_bf16, int32_t n_blocks,
                        int32_t R, const void* kpool, const int32_t* tables, double* out) {
  const int32_t T = n_blocks * b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < (int64_t)R * H; unit++) {
    const int32_t r = (int32_t)(unit / H), h = (int32_t)(unit % H);
    double* K = (double*)malloc((size_t)T * d * sizeof(double));
    double* nrm = (double*)malloc((size_t)T * sizeof(double));
    for (int32_t j = 0; j < T; j++) {
      size_t base = row_index(tables[(size_t)r * n_blocks + j / b], h, j % b, H, b, d);
      double ss = 0.0;
      for (int32_t e = 0; e < d; e++) {
        K[(size_t)j * d + e] = widen(kpool, base + e, is_bf16);
        ss += K[(size_t)j * d + e] * K[(size_t)j * d + e];
      }
      nrm[j] = sqrt(ss);
    }
    for (int32_t a = 0; a < T; a++) {
      double acc = 0.0;
      for (int32_t c = 0; c < T; c++) {
        if (c == a || nrm[a] == 0.0 || nrm[c] == 0.0) continue;
        double dot = 0.0;
        for (int32_t e = 0; e < d; e++) dot += K[(size_t)a * d + e] * K[(size_t)c * d + e];
        acc += dot / (nrm[a] * nrm[c]);
      }
      out[((size_t)r * H + h) * T + a] = acc / (double)(T - 1);
    }
    free(K);
    free(nrm);
  }
}
