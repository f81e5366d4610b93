/*
 * Plain CPU oracle for the sparse-attention indexer hot path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, by the package smoke check
 * and by the benchmark's CPU-baseline leg, never by the library.  It shares
 * no code with the HIP path.  Slow on purpose: every function is the plain
 * definition, or the pages' steps in the pages' order, written out.
 *
 * Sources (cited by page title and section):
 *   [DoSA]    "DoSA: reducing the indexer's full scoring with safe upper
 *             bounds" (notes.kuangjux.top, DoSA reading notes).
 *   [WIT]     "Segment Witnesses" (teerth.dev, Aether-Lang kvwitness).
 *   [BLOCK]   ferrox_core block_sparse.rs (docs.rs, ferrox-core 0.14.0).
 *   [OCP-FP8] OCP 8-bit floating point specification, E4M3 encoding.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int32_t orc_num_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Element decoding                                                          */
/* ------------------------------------------------------------------------ */

/* [OCP-FP8] E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, S.1111.111 is NaN, largest finite 448.  Subnormals
 * (exponent field 0) are m * 2^-9. */
double orc_e4m3fn_to_double(uint8_t b) {
  int sign = b >> 7;
  int e = (b >> 3) & 0xF;
  int m = b & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double orc_decode(const void* p, int32_t dtype, int64_t i) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: return bf16_to_double(((const uint16_t*)p)[i]);
    case ORC_FP8_E4M3FN: return orc_e4m3fn_to_double(((const uint8_t*)p)[i]);
    default: return NAN;
  }
}

/* ------------------------------------------------------------------------ */
/* Lightning-indexer score and top-K                                          */
/* ------------------------------------------------------------------------ */

/* Row r sees keys [off, off + vis): the query sits at the last visible
 * position ([WIT] "Implementation rule and contracts", Coordinates row).
 * Out-of-range lengths or offsets are clamped so nothing outside k is read. */
int64_t orc_visible(const orc_problem* P, int32_t r) {
  int64_t off = P->k_row_offset ? P->k_row_offset[r] : 0;
  int64_t v = P->vis_len[r];
  if (off < 0 || off > P->n_k) return 0;
  if (v < 0) v = 0;
  if (v > P->max_vis) v = P->max_vis;
  if (v > P->n_k - off) v = P->n_k - off;
  return v;
}

/* Dequantised key j of the key store, widened exactly to double; an fp8 key
 * is the decoded byte times its per-token scale. */
static double load_key(const orc_problem* P, int64_t key, double* kd) {
  double sc = (P->k_dtype == ORC_FP8_E4M3FN) ? (double)P->k_scale[key] : 1.0;
  double nn = 0.0;
  for (int d = 0; d < P->D; ++d) {
    kd[d] = orc_decode(P->k, P->k_dtype, key * P->D + d) * sc;
    nn += kd[d] * kd[d];
  }
  return sqrt(nn);
}

static void load_query(const orc_problem* P, int32_t r, double* qd, double* qn) {
  for (int h = 0; h < P->H; ++h) {
    double nn = 0.0;
    for (int d = 0; d < P->D; ++d) {
      double x = orc_decode(P->q, P->q_dtype, ((int64_t)r * P->H + h) * P->D + d);
      qd[h * P->D + d] = x;
      nn += x * x;
    }
    qn[h] = sqrt(nn);
  }
}

static double dotd(const double* a, const double* b, int D) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) s += a[d] * b[d];
  return s;
}

/* [DoSA] section 3: s(k) = sum_h w_h [q_h . k]_+ with [x]_+ = max(x, 0).  All
 * query heads share one index key; weights are signed; a negative dot is
 * clipped to zero before its weight applies, so it never deducts.  x[] gets
 * the per-head dots (may be NULL). */
static double score_key(const double* qd, const double* qn, const float* w, int H, int D,
                        const double* kd, double knorm, double* x, double* m_out,
                        double* n_out) {
  double s = 0.0, m = 0.0, n = 0.0;
  for (int h = 0; h < H; ++h) {
    double xh = dotd(qd + (int64_t)h * D, kd, D);
    double a = xh > 0.0 ? xh : 0.0;
    double wh = (double)w[h];
    if (x) x[h] = xh;
    s += wh * a;
    m += fabs(wh) * a;
    n += fabs(wh) * qn[h] * knorm;
  }
  if (m_out) *m_out = m;
  if (n_out) *n_out = n;
  return s;
}

int64_t orc_score_row(const orc_problem* P, int32_t r, double* s, double* m, double* n) {
  const int H = P->H, D = P->D;
  const int64_t v = orc_visible(P, r);
  const int64_t off = P->k_row_offset ? P->k_row_offset[r] : 0;
  const float* w = P->w + (int64_t)r * P->w_row_stride;
  double* qd = (double*)malloc(sizeof(double) * H * D);
  double* qn = (double*)malloc(sizeof(double) * H);
  double* kd = (double*)malloc(sizeof(double) * (D > 0 ? D : 1));
  load_query(P, r, qd, qn);
  for (int64_t j = 0; j < v; ++j) {
    double knorm = load_key(P, off + j, kd);
    double mm, nn;
    double ss = score_key(qd, qn, w, H, D, kd, knorm, NULL, &mm, &nn);
    if (s) s[j] = ss;
    if (m) m[j] = mm;
    if (n) n[j] = nn;
  }
  free(qd);
  free(qn);
  free(kd);
  return v;
}

typedef struct {
  double s;
  int32_t id;
} scored_id;

/* One total order for every selection: score descending, then id ascending.
 * -0 and +0 compare equal here and fall through to the id ([DoSA] section 1:
 * tied IDs only agree under one consistent total order). */
static int cmp_score_desc_id_asc(const void* pa, const void* pb) {
  const scored_id* a = (const scored_id*)pa;
  const scored_id* b = (const scored_id*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

int32_t orc_topk(const double* s, const int32_t* ids, int64_t n, int32_t K, int32_t* out_idx,
                 double* out_score) {
  if (K <= 0) return 0;
  scored_id* a = (scored_id*)malloc(sizeof(scored_id) * (n > 0 ? n : 1));
  for (int64_t j = 0; j < n; ++j) {
    a[j].s = s[j];
    a[j].id = ids ? ids[j] : (int32_t)j;
  }
  qsort(a, (size_t)n, sizeof(scored_id), cmp_score_desc_id_asc);
  int32_t cnt = (int32_t)(n < K ? n : K);
  for (int32_t t = 0; t < K; ++t) {
    if (out_idx) out_idx[t] = t < cnt ? a[t].id : -1;
    if (out_score) out_score[t] = t < cnt ? a[t].s : -INFINITY;
  }
  free(a);
  return cnt;
}

void orc_idx_score_topk_rows(const orc_problem* P, const int32_t* rows, int32_t n_rows,
                             int32_t* out_idx, double* out_score, double* s_rows,
                             double* m_rows, double* n_rows_out, int64_t row_stride) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    int32_t r = rows[i];
    int64_t cap = P->max_vis > 0 ? P->max_vis : 1;
    double* s = (double*)malloc(sizeof(double) * cap);
    double* m = m_rows ? m_rows + (int64_t)i * row_stride : NULL;
    double* n = n_rows_out ? n_rows_out + (int64_t)i * row_stride : NULL;
    int64_t v = orc_score_row(P, r, s, m, n);
    if (s_rows) memcpy(s_rows + (int64_t)i * row_stride, s, sizeof(double) * v);
    orc_topk(s, NULL, v, P->topk, out_idx ? out_idx + (int64_t)i * P->topk : NULL,
             out_score ? out_score + (int64_t)i * P->topk : NULL);
    free(s);
  }
}

/* ------------------------------------------------------------------------ */
/* Segment witnesses ([WIT])                                                  */
/* ------------------------------------------------------------------------ */

#define ORC_MAX_SEGMENTS 64 /* [WIT] "Refusals": 64-bit occupancy mask bound */

/* [WIT] "Object": sigma(x) = floor(x * S_eff / L), S_eff = min(S, L).
 * "Rust API" notes: a context length of 0 is read as 1. */
int64_t orc_segment_of(int64_t token, int64_t context_len, int64_t num_segments) {
  int64_t L = context_len < 1 ? 1 : context_len;
  int64_t Se = num_segments < L ? num_segments : L;
  return token * Se / L;
}

/* [WIT] "Object": left edge e_s = ceil(s * L / S_eff). */
int64_t orc_segment_edge(int64_t s, int64_t L, int64_t S_eff) {
  return (s * L + S_eff - 1) / S_eff;
}

/* [WIT] "Implementation rule and contracts", Out-of-range row: an entry
 * x >= L marks segment min(floor(x * S_eff / L), S - 1); in-range entries
 * mark sigma(x).  Negative entries are padding (callers skip them). */
int64_t orc_occupied_segment(int64_t x, int64_t L, int64_t S) {
  int64_t Se = S < L ? S : L;
  int64_t seg = x * Se / L;
  if (x >= L && seg > S - 1) seg = S - 1;
  return seg;
}

/* Witnesses of one row, ascending segment order: e_s for every s < S_eff that
 * no learned entry occupies ([WIT] "Object", W(K)).  Returns the count. */
static int32_t row_witnesses(const int32_t* row, int32_t topk, int64_t L, int32_t S,
                             int32_t* wit) {
  unsigned char occ[ORC_MAX_SEGMENTS];
  if (L <= 0) return 0; /* "Fallback": no witnesses for L <= 0 */
  int64_t Se = S < L ? S : L;
  memset(occ, 0, sizeof occ);
  for (int32_t t = 0; t < topk; ++t) {
    int64_t x = row[t];
    if (x < 0) continue; /* -1 padding marks no segment */
    occ[orc_occupied_segment(x, L, S)] = 1;
  }
  int32_t n = 0;
  for (int64_t s = 0; s < Se; ++s)
    if (!occ[s]) wit[n++] = (int32_t)orc_segment_edge(s, L, Se);
  return n;
}

/* [WIT] "Rust API": topology_witness_indices, row-major [rows, S], -1 where a
 * segment is occupied or does not exist.  Refuses S == 0 or S > 64. */
int32_t orc_witness_indices(const int32_t* learned, int32_t rows, int32_t topk,
                            const int32_t* context_lens, int32_t num_segments, int32_t* out) {
  if (rows < 0 || topk < 0) return ORC_INVALID_ARGUMENT;
  if (rows > 0 && !context_lens) return ORC_ROWS_MISMATCH;
  if (num_segments <= 0 || num_segments > ORC_MAX_SEGMENTS) return ORC_SEGMENTS_OUT_OF_RANGE;
  for (int32_t r = 0; r < rows; ++r) {
    unsigned char occ[ORC_MAX_SEGMENTS];
    int64_t L = context_lens[r];
    for (int32_t s = 0; s < num_segments; ++s) out[(int64_t)r * num_segments + s] = -1;
    if (L <= 0) continue;
    int64_t Se = num_segments < L ? num_segments : L;
    memset(occ, 0, sizeof occ);
    for (int32_t t = 0; t < topk; ++t) {
      int64_t x = learned[(int64_t)r * topk + t];
      if (x >= 0) occ[orc_occupied_segment(x, L, num_segments)] = 1;
    }
    for (int64_t s = 0; s < Se; ++s)
      if (!occ[s]) out[(int64_t)r * num_segments + s] = (int32_t)orc_segment_edge(s, L, Se);
  }
  return ORC_OK;
}

/* [WIT] "Implementation rule and contracts": slots [0, keep) are kept
 * verbatim; witnesses in ascending segment order overwrite keep, keep+1, ...
 * up to B = min(max_replacements, topk - keep); extra witnesses are dropped.
 * Occupancy is read from the whole learned row before any slot is written
 * ("Caveats").  Checks run before anything is written ("Refusals": a
 * refused call leaves the buffer untouched); S == 0, B == 0 or zero rows is
 * the identity ("Disabled" row). */
int32_t orc_kvwitness_merge(int32_t* topk_idx, int32_t rows, int32_t topk,
                            const int32_t* context_lens, int32_t num_segments, int32_t keep,
                            int32_t max_replacements) {
  if (rows < 0 || topk < 0 || keep < 0 || max_replacements < 0) return ORC_INVALID_ARGUMENT;
  if (rows > 0 && !context_lens) return ORC_ROWS_MISMATCH;
  if (rows > 0 && topk > 0 && !topk_idx) return ORC_INVALID_ARGUMENT;
  if (num_segments < 0 || num_segments > ORC_MAX_SEGMENTS) return ORC_SEGMENTS_OUT_OF_RANGE;
  if (keep > topk) return ORC_KEEP_OUT_OF_RANGE;
  int32_t B = max_replacements < topk - keep ? max_replacements : topk - keep;
  if (num_segments == 0 || B == 0 || rows == 0) return ORC_OK;
  for (int32_t r = 0; r < rows; ++r) {
    int32_t wit[ORC_MAX_SEGMENTS];
    int32_t* row = topk_idx + (int64_t)r * topk;
    int32_t n = row_witnesses(row, topk, context_lens[r], num_segments, wit);
    for (int32_t i = 0; i < n && i < B; ++i) row[keep + i] = wit[i];
  }
  return ORC_OK;
}

/* [WIT] "Null models and metrics": coverage(C) = |{sigma(x) : x in C, 0 <= x < L}|
 * / S_eff; 1 when there are no segments.  Padding, duplicates and out-of-range
 * entries count for nothing. */
double orc_segment_coverage(const int32_t* cand, int32_t n, int64_t L, int64_t num_segments) {
  unsigned char seen[ORC_MAX_SEGMENTS];
  if (L <= 0 || num_segments <= 0) return 1.0;
  int64_t Se = num_segments < L ? num_segments : L;
  if (Se > ORC_MAX_SEGMENTS) return NAN;
  memset(seen, 0, sizeof seen);
  int64_t hit = 0;
  for (int32_t i = 0; i < n; ++i) {
    int64_t x = cand[i];
    if (x < 0 || x >= L) continue;
    int64_t s = x * Se / L;
    if (!seen[s]) {
      seen[s] = 1;
      ++hit;
    }
  }
  return (double)hit / (double)Se;
}

/* ------------------------------------------------------------------------ */
/* Block-sparse selection ([BLOCK])                                           */
/* ------------------------------------------------------------------------ */

/* [BLOCK] module docs, "Four rules": a block is scored by the raw dot
 * product of the index query and a position's index key, with no scale.  The
 * page's dot helper sums f32 products in index order: each product is rounded
 * to f32 and then added (no fused multiply-add), starting from +0.0f, so the
 * result is never -0. */
float orc_block_dot(const float* a, const float* b, int32_t D) {
  float acc = 0.0f;
  for (int32_t d = 0; d < D; ++d) {
    float p = a[d] * b[d];
    acc = acc + p;
  }
  return acc;
}

/* [BLOCK] the configuration's causal block count: the blocks covering
 * positions 0..=query_pos; 0 when the block size is 0.  A negative position
 * sees no block. */
int64_t orc_causal_blocks(int64_t query_pos, int64_t block_size) {
  if (block_size <= 0 || query_pos < 0) return 0;
  return query_pos / block_size + 1;
}

/* [BLOCK] the order of block scores: higher score first; equal scores go to
 * the lower block (the selection's comment on deterministic ties).  Scores
 * are never NaN and never -0 here, where the IEEE comparison is the page's
 * total order. */
static int block_before(float sa, int64_t a, float sb, int64_t b) {
  return sa > sb || (sa == sb && a < b);
}

/* [BLOCK] the public selection entry's doc comment and the module docs
 * ("Four rules"), for one query position, stated as a set:
 *   n   = min(causal blocks, ceil(n_pos / bs))   (a query cannot see past
 *         the keys that exist); n == 0 gives empty selections;
 *   F   = the first min(init, n) blocks and the last min(local, n) blocks,
 *         force-included before any scoring;
 *   B   = max(top, |F|), the budget counting the forced blocks;
 *   per KV head h, every other block b gets score(b) = the MAX over its
 *         causally visible positions [b bs, min((b+1) bs, n_pos, pos+1)) of
 *         the dot above;
 *   the selection is F plus the non-forced blocks whose rank under the
 *         order above is below B - |F| (a block's rank = the number of
 *         non-forced blocks ordered before it), written ascending.
 * Its size is min(n, B).  Returns 0, or -1 if `width` cannot hold a
 * selection. */
int32_t orc_block_select_query(const float* q, const float* k, int64_t query_pos, int32_t H,
                               int32_t D, int64_t n_pos, int32_t block_size, int32_t top_blocks,
                               int32_t init_blocks, int32_t local_blocks, int32_t* out,
                               int32_t width, int32_t* counts, float* block_scores) {
  int64_t n = orc_causal_blocks(query_pos, block_size);
  int64_t exist = block_size > 0 ? (n_pos + block_size - 1) / block_size : 0;
  if (exist < n) n = exist;
  for (int32_t h = 0; h < H; ++h) {
    counts[h] = 0;
    for (int32_t t = 0; t < width; ++t) out[(int64_t)h * width + t] = -1;
  }
  if (n <= 0) return 0;
  unsigned char* forced = (unsigned char*)calloc((size_t)n, 1);
  float* score = (float*)malloc(sizeof(float) * (size_t)n);
  for (int64_t b = 0; b < n; ++b)
    forced[b] = (b < init_blocks) || (b >= n - local_blocks);
  int64_t nf = 0;
  for (int64_t b = 0; b < n; ++b) nf += forced[b];
  const int64_t budget = top_blocks > nf ? top_blocks : nf;
  const int64_t free_slots = budget - nf; /* non-forced blocks that join */
  int32_t rc = 0;
  for (int32_t h = 0; h < H && rc == 0; ++h) {
    const float* qh = q + (int64_t)h * D;
    if (free_slots > 0) {
      for (int64_t b = 0; b < n; ++b) {
        if (forced[b]) continue;
        int64_t end = (b + 1) * block_size;
        if (end > n_pos) end = n_pos;
        if (end > query_pos + 1) end = query_pos + 1;
        float best = -INFINITY;
        for (int64_t p = b * block_size; p < end; ++p) {
          float v = orc_block_dot(qh, k + p * D, D);
          if (v > best) best = v;
        }
        score[b] = best;
        if (block_scores) block_scores[(int64_t)h * n + b] = best;
      }
    }
    int64_t c = 0;
    for (int64_t b = 0; b < n; ++b) {
      int in = forced[b];
      if (!in && free_slots > 0) {
        int64_t rank = 0;
        for (int64_t o = 0; o < n && rank < free_slots; ++o)
          if (!forced[o] && block_before(score[o], o, score[b], b)) ++rank;
        in = rank < free_slots;
      }
      if (!in) continue;
      if (c >= width) {
        rc = -1;
        break;
      }
      out[(int64_t)h * width + c++] = (int32_t)b;
    }
    counts[h] = (int32_t)c;
  }
  free(forced);
  free(score);
  return rc;
}

void orc_block_select_rows(const float* q, const float* k, const int64_t* query_pos,
                           const int32_t* rows, int32_t n_rows, int32_t H, int32_t D,
                           int64_t n_pos, int32_t block_size, int32_t top_blocks,
                           int32_t init_blocks, int32_t local_blocks, int32_t* out,
                           int32_t width, int32_t* counts) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    int32_t r = rows[i];
    orc_block_select_query(q + (int64_t)r * H * D, k, query_pos[r], H, D, n_pos, block_size,
                           top_blocks, init_blocks, local_blocks,
                           out + (int64_t)i * H * width, width, counts + (int64_t)i * H, NULL);
  }
}

/* [BLOCK] the doc comment of the positions helper: the positions a block
 * selection covers, ascending, causally clipped, deduplicated.  Returns the count written to out.  A negative
 * entry is the -1 padding of an i32 block list and covers nothing (the
 * page's lists are unsigned and unpadded). */
int64_t orc_positions_of_blocks(const int32_t* blocks, int32_t n_sel, int64_t query_pos,
                                int64_t n_pos, int32_t block_size, int64_t* out) {
  int64_t n = 0;
  for (int32_t i = 0; i < n_sel; ++i) {
    if (blocks[i] < 0) continue;
    int64_t start = (int64_t)blocks[i] * block_size;
    int64_t end = start + block_size;
    if (end > n_pos) end = n_pos;
    if (end > query_pos + 1) end = query_pos + 1;
    for (int64_t p = start; p < end; ++p) out[n++] = p;
  }
  /* insertion sort + dedup: sizes here are tiny */
  for (int64_t i = 1; i < n; ++i) {
    int64_t v = out[i], j = i - 1;
    while (j >= 0 && out[j] > v) {
      out[j + 1] = out[j];
      --j;
    }
    out[j + 1] = v;
  }
  int64_t m = 0;
  for (int64_t i = 0; i < n; ++i)
    if (m == 0 || out[m - 1] != out[i]) out[m++] = out[i];
  return m;
}

/* positions_of_blocks over [n_q, n_heads, width] block lists (query q's
 * lists share query_pos[q]): list l's positions as i32 in out[l * out_width
 * ..], -1 after the count[l] covered ones.  out_width must hold every
 * position the list can cover. */
void orc_positions_of_block_rows(const int32_t* blocks, int32_t n_q, int32_t n_heads,
                                 int32_t width, const int64_t* query_pos, int64_t n_pos,
                                 int32_t block_size, int32_t* out, int64_t out_width,
                                 int32_t* count) {
  int64_t* tmp = (int64_t*)malloc(sizeof(int64_t) * (size_t)(width * (int64_t)block_size + 1));
  for (int64_t l = 0; l < (int64_t)n_q * n_heads; ++l) {
    int64_t m = orc_positions_of_blocks(blocks + l * width, width, query_pos[l / n_heads], n_pos,
                                        block_size, tmp);
    for (int64_t i = 0; i < out_width; ++i) out[l * out_width + i] = i < m ? (int32_t)tmp[i] : -1;
    count[l] = (int32_t)m;
  }
  free(tmp);
}

/* Gather slots for the attention that consumes a selection row.  [WIT]
 * Coordinates: entries are row-relative offsets with valid range [0, L_r);
 * -1 is padding, and a learned entry >= L_r passes through the merge but
 * names no token of the row.  So entry x of row r is gathered iff
 * 0 <= x < L_r, and every other entry maps to -1.  A gathered x lives at
 *   row_start[r] + x                                  (flat KV buffer), or
 *   page_table[r][x / page_size] * page_size + x % page_size   (paged KV: a
 *   page holds page_size consecutive tokens; [BLOCK] module docs make the
 *   128-token block the KV page),
 * and -1 when x's page lies past pages_per_row or its page id is negative.
 * Exactly one of row_start / page_table is non-NULL. */
void orc_gather_slots(const int32_t* idx, int32_t rows, int32_t width, const int32_t* lens,
                      const int64_t* row_start, const int32_t* page_table, int32_t pages_per_row,
                      int32_t page_size, int64_t* out) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t i = 0; i < width; ++i) {
      const int64_t x = idx[r * width + i];
      int64_t slot = -1;
      if (x >= 0 && x < (int64_t)lens[r]) {
        if (row_start) {
          slot = row_start[r] + x;
        } else {
          const int64_t pg = x / page_size;
          if (pg < pages_per_row) {
            const int64_t id = page_table[r * pages_per_row + pg];
            if (id >= 0) slot = id * page_size + x % page_size;
          }
        }
      }
      out[r * width + i] = slot;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* DoSA certified prune ([DoSA])                                              */
/* ------------------------------------------------------------------------ */

static int cmp_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* Seeds must be visible to every row: the common visible prefix [0, c). */
int32_t orc_dosa_common_prefix(const orc_problem* P) {
  int64_t c = -1;
  for (int32_t r = 0; r < P->n_q; ++r) {
    int64_t v = orc_visible(P, r);
    if (c < 0 || v < c) c = v;
  }
  return (int32_t)(c < 0 ? 0 : c);
}

/* [DoSA] section 4, cold prior: representative queries evenly spaced over
 * the chunk, first and last included: t_i = round(i (n_q - 1) / (R - 1)). */
int32_t orc_dosa_rep_row(int32_t i, int32_t n_rep, int32_t n_q) {
  if (n_rep <= 1 || n_q <= 1) return 0;
  int64_t num = 2 * (int64_t)i * (n_q - 1) + (n_rep - 1);
  return (int32_t)(num / (2 * (int64_t)(n_rep - 1)));
}

/* [DoSA] section 4 (cold prior): fully score the representative queries over
 * the common visible prefix, count how often each key appears in their top
 * rep_topk lists, and take n_seeds keys by (count desc, key asc).  Seeds are
 * returned ascending.  Refuses (ORC_NOT_ENOUGH_KEYS) when the prefix is
 * shorter than n_seeds or n_seeds < K (the threshold needs >= K keys,
 * section 2 step 1). */
int32_t orc_dosa_seeds(const orc_problem* P, const orc_dosa_params* dp, int32_t* seeds,
                       int32_t* counts) {
  int32_t c = orc_dosa_common_prefix(P);
  if (dp->n_seeds > c || dp->n_seeds < P->topk || dp->n_seeds <= 0) return ORC_NOT_ENOUGH_KEYS;
  int32_t R = dp->n_rep_queries;
  int32_t* cnt = (int32_t*)calloc((size_t)c, sizeof(int32_t));
  double* s = (double*)malloc(sizeof(double) * (P->max_vis > 0 ? P->max_vis : 1));
  int32_t* top = (int32_t*)malloc(sizeof(int32_t) * (dp->rep_topk > 0 ? dp->rep_topk : 1));
  for (int32_t i = 0; i < R; ++i) {
    int32_t t = orc_dosa_rep_row(i, R, P->n_q);
    orc_score_row(P, t, s, NULL, NULL);
    int32_t n = orc_topk(s, NULL, c, dp->rep_topk, top, NULL);
    for (int32_t j = 0; j < n; ++j) cnt[top[j]] += 1;
  }
  int32_t ns = 0;
  for (int32_t v = R; v >= 0 && ns < dp->n_seeds; --v)
    for (int32_t j = 0; j < c && ns < dp->n_seeds; ++j)
      if (cnt[j] == v) seeds[ns++] = j;
  qsort(seeds, (size_t)ns, sizeof(int32_t), cmp_i32);
  if (counts) memcpy(counts, cnt, sizeof(int32_t) * c);
  free(cnt);
  free(s);
  free(top);
  return ORC_OK;
}

typedef struct {
  double imp;
  int32_t h;
} head_rank;

static int cmp_head_rank(const void* pa, const void* pb) {
  const head_rank* a = (const head_rank*)pa;
  const head_rank* b = (const head_rank*)pb;
  if (a->imp > b->imp) return -1;
  if (a->imp < b->imp) return 1;
  return (a->h > b->h) - (a->h < b->h);
}

int64_t orc_dosa_head_dots(int64_t n_seeds, int64_t n_scanned, int64_t filter_dots_per_key,
                           int64_t n_survivors, int32_t H) {
  /* [DoSA] section 5 accounting: full-head dots for seeds and survivors,
   * filter dots for every scanned key. */
  return n_seeds * H + n_scanned * filter_dots_per_key + n_survivors * H;
}

static void full_row_topk(const orc_problem* P, int32_t r, int32_t* out_idx, double* out_score) {
  double* s = (double*)malloc(sizeof(double) * (P->max_vis > 0 ? P->max_vis : 1));
  int64_t v = orc_score_row(P, r, s, NULL, NULL);
  orc_topk(s, NULL, v, P->topk, out_idx, out_score);
  free(s);
}

/* [DoSA] section 2, for one prefill row r:
 *  1. seeds: score every seed with all heads; tau = K-th highest seed score;
 *     keep the seeds' top-K.  tau stays fixed for the rest of the row.
 *  2. for every other visible key, a safe upper bound U built from
 *     (section 3.1) kept heads' exact activations, omitted positive heads
 *     bounded through one kept anchor, q_h = beta q_j + d_h with beta >= 0:
 *     [q_h.k]_+ <= beta [q_j.k]_+ + |d_h| |k|, and
 *     (section 3.2) omitted negative heads active on at least neg_active_frac
 *     of the sampled seeds aggregated as a_A = sum |w_h| q_h, deducting [a_A.k]_+,
 *     which never exceeds their true deduction.
 *     A key is excluded iff U < tau (U == tau is kept).
 *  3. survivors get their exact score; those below tau are dropped; the final
 *     top-K is taken over the seeds' top-K plus the kept survivors, by score.
 * Planning choices the pages leave open: activation statistics come from a
 * 128-seed sample (section 4 samples 128 positions of the seed region); the
 * kept heads are the kept_heads largest |w_h| * mean [x_h]_+ over the sample
 * (ties: lower head); an omitted positive head anchors on the kept
 * head with the smallest residual under the clamped projection
 * beta = max(0, q_h.q_j / |q_j|^2) (ties: lower head).  The bound carries a
 * 1e-9 * sum_h |w_h| |q_h| |k| margin so double rounding can never make it
 * undercut the score.  More survivors than survivor_capacity (when >= 0)
 * sends the row to the exact unpruned path ([DoSA] section 4: error states
 * trigger an exact recovery). */
int32_t orc_dosa_row(const orc_problem* P, const orc_dosa_params* dp, const int32_t* seeds,
                     int32_t r, int32_t* out_idx, double* out_score, orc_dosa_row_stats* st,
                     const orc_dosa_diag* dg) {
  const int H = P->H, D = P->D, K = P->topk;
  const int32_t ns = dp->n_seeds;
  const int64_t v = orc_visible(P, r);
  const float* w = P->w + (int64_t)r * P->w_row_stride;
  orc_dosa_row_stats loc;
  memset(&loc, 0, sizeof loc);
  loc.tau = NAN;
  if (dg && dg->pos_part)
    for (int64_t j = 0; j < v; ++j) dg->pos_part[j] = NAN;
  if (dg && dg->neg_part)
    for (int64_t j = 0; j < v; ++j) dg->neg_part[j] = NAN;
  if (dg && dg->U)
    for (int64_t j = 0; j < v; ++j) dg->U[j] = NAN;

  int bad = (seeds == NULL) || (ns < K) || (ns <= 0) || (P->k_row_offset != NULL);
  for (int32_t i = 0; !bad && i < ns; ++i)
    if (seeds[i] < 0 || seeds[i] >= v || (i > 0 && seeds[i] <= seeds[i - 1])) bad = 1;
  if (bad) {
    full_row_topk(P, r, out_idx, out_score);
    loc.fallback = 1;
    if (st) *st = loc;
    return ORC_OK;
  }

  double* qd = (double*)malloc(sizeof(double) * H * D);
  double* qn = (double*)malloc(sizeof(double) * H);
  double* kd = (double*)malloc(sizeof(double) * D);
  double* x = (double*)malloc(sizeof(double) * H);
  double* seed_s = (double*)malloc(sizeof(double) * ns);
  double* act = (double*)calloc((size_t)H, sizeof(double));
  double* relu_mean = (double*)calloc((size_t)H, sizeof(double));
  unsigned char* is_seed = (unsigned char*)calloc((size_t)(v > 0 ? v : 1), 1);
  int32_t* seed_top = (int32_t*)malloc(sizeof(int32_t) * K);
  double* seed_top_s = (double*)malloc(sizeof(double) * K);
  load_query(P, r, qd, qn);

  /* Step 1: the seed threshold.  The activation statistics come from a
   * sample of the seeds ([DoSA] section 4: the planner counts activation
   * patterns over 128 positions of the seed region): m = min(128, ns) seeds
   * evenly spaced in seed order, seed index round(i (ns - 1) / (m - 1)). */
  const int32_t m = ns < 128 ? ns : 128;
  int32_t next_sample = 0, si = 0;  /* the next sample's seed index, and its i */
  for (int32_t i = 0; i < ns; ++i) {
    int64_t j = seeds[i];
    is_seed[j] = 1;
    double knorm = load_key(P, j, kd);
    seed_s[i] = score_key(qd, qn, w, H, D, kd, knorm, x, NULL, NULL);
    if (si < m && i == next_sample) {
      for (int h = 0; h < H; ++h) {
        if (x[h] > 0.0) {
          act[h] += 1.0;
          relu_mean[h] += x[h];
        }
      }
      ++si;
      next_sample = m > 1 ? (int32_t)((2LL * si * (ns - 1) + (m - 1)) / (2LL * (m - 1))) : ns;
    }
  }
  for (int h = 0; h < H; ++h) {
    act[h] /= m;
    relu_mean[h] /= m;
  }
  orc_topk(seed_s, seeds, ns, K, seed_top, seed_top_s);
  const double tau = seed_top_s[K - 1];
  loc.tau = tau;

  /* Plan: kept heads, anchors, folded weights, residual, negative aggregate. */
  int32_t kept = dp->kept_heads < H ? dp->kept_heads : H;
  if (kept < 0) kept = 0;
  head_rank* hr = (head_rank*)malloc(sizeof(head_rank) * H);
  for (int h = 0; h < H; ++h) {
    hr[h].imp = fabs((double)w[h]) * relu_mean[h];
    hr[h].h = h;
  }
  qsort(hr, (size_t)H, sizeof(head_rank), cmp_head_rank);
  int32_t* role = (int32_t*)calloc((size_t)H, sizeof(int32_t));
  int32_t* anchor = (int32_t*)malloc(sizeof(int32_t) * H);
  double* beta = (double*)calloc((size_t)H, sizeof(double));
  double* dnorm = (double*)calloc((size_t)H, sizeof(double));
  double* wfold = (double*)calloc((size_t)H, sizeof(double));
  double* a_agg = (double*)calloc((size_t)D, sizeof(double));
  double* dvec = (double*)malloc(sizeof(double) * D);
  for (int h = 0; h < H; ++h) anchor[h] = -1;
  for (int32_t i = 0; i < kept; ++i) role[hr[i].h] = 1;
  for (int h = 0; h < H; ++h)
    if (role[h] == 1) wfold[h] = (double)w[h];
  double R = 0.0;
  for (int h = 0; h < H; ++h) {
    if (role[h] == 1) continue;
    const double* qh = qd + (int64_t)h * D;
    if (w[h] > 0.0f) {
      role[h] = 2;
      double best_r2 = INFINITY, best_beta = 0.0;
      int best_j = -1;
      for (int j = 0; j < H; ++j) {
        if (role[j] != 1) continue;
        const double* qj = qd + (int64_t)j * D;
        double qq = dotd(qj, qj, D);
        double b = qq > 0.0 ? dotd(qh, qj, D) / qq : 0.0;
        if (b < 0.0) b = 0.0;
        for (int d = 0; d < D; ++d) dvec[d] = qh[d] - b * qj[d];
        double r2 = dotd(dvec, dvec, D);
        if (r2 < best_r2) {
          best_r2 = r2;
          best_beta = b;
          best_j = j;
        }
      }
      if (best_j < 0) { /* no kept head: the residual is the whole query */
        best_beta = 0.0;
        best_r2 = dotd(qh, qh, D);
      }
      anchor[h] = best_j;
      beta[h] = best_beta;
      dnorm[h] = sqrt(best_r2);
      if (best_j >= 0) wfold[best_j] += (double)w[h] * best_beta;
      R += (double)w[h] * dnorm[h];
      loc.n_pos_omitted++;
    } else if (w[h] < 0.0f) {
      if (act[h] >= dp->neg_active_frac) {
        role[h] = 3;
        for (int d = 0; d < D; ++d) a_agg[d] += fabs((double)w[h]) * qh[d];
        loc.n_neg_aggregated++;
      } else {
        role[h] = 4;
        loc.n_neg_dropped++;
      }
    }
  }
  loc.n_kept_heads = kept;
  loc.R = R;

  /* Steps 2-3: bound scan, exact rescoring of survivors. */
  double* cand_s = (double*)malloc(sizeof(double) * (K + (v > 0 ? v : 1)));
  int32_t* cand_id = (int32_t*)malloc(sizeof(int32_t) * (K + (v > 0 ? v : 1)));
  int64_t nc = 0;
  for (int32_t t = 0; t < K; ++t) {
    cand_s[nc] = seed_top_s[t];
    cand_id[nc] = seed_top[t];
    ++nc;
  }
  for (int64_t j = 0; j < v; ++j) {
    if (is_seed[j]) continue;
    loc.n_scanned++;
    double knorm = load_key(P, j, kd);
    double pos = R * knorm, ntol = 0.0;
    for (int h = 0; h < H; ++h) {
      ntol += fabs((double)w[h]) * qn[h] * knorm;
      if (role[h] != 1) continue;
      double xh = dotd(qd + (int64_t)h * D, kd, D);
      pos += wfold[h] * (xh > 0.0 ? xh : 0.0);
    }
    double xa = dotd(a_agg, kd, D);
    double neg = xa > 0.0 ? xa : 0.0;
    double U = pos - neg + 1e-9 * ntol;
    if (dg && dg->pos_part) dg->pos_part[j] = pos;
    if (dg && dg->neg_part) dg->neg_part[j] = neg;
    if (dg && dg->U) dg->U[j] = U;
    if (!(U >= tau)) continue; /* excluded only when U < tau */
    loc.n_survivors++;
    double s = score_key(qd, qn, w, H, D, kd, knorm, NULL, NULL, NULL);
    if (s >= tau) {
      cand_s[nc] = s;
      cand_id[nc] = (int32_t)j;
      ++nc;
      loc.n_kept_survivors++;
    }
  }
  loc.head_dots = orc_dosa_head_dots(ns, loc.n_scanned, kept + (loc.n_neg_aggregated > 0),
                                     loc.n_survivors, H);
  if (dp->survivor_capacity >= 0 && loc.n_survivors > dp->survivor_capacity) {
    full_row_topk(P, r, out_idx, out_score);
    loc.fallback = 1;
  } else {
    orc_topk(cand_s, cand_id, nc, K, out_idx, out_score);
  }

  if (dg) {
    for (int h = 0; h < H; ++h) {
      if (dg->head_role) dg->head_role[h] = role[h];
      if (dg->anchor) dg->anchor[h] = anchor[h];
      if (dg->beta) dg->beta[h] = beta[h];
      if (dg->dnorm) dg->dnorm[h] = dnorm[h];
      if (dg->wfold) dg->wfold[h] = wfold[h];
      if (dg->act) dg->act[h] = act[h];
    }
    if (dg->a_agg) memcpy(dg->a_agg, a_agg, sizeof(double) * D);
  }
  if (st) *st = loc;
  free(qd); free(qn); free(kd); free(x); free(seed_s); free(act); free(relu_mean);
  free(is_seed); free(seed_top); free(seed_top_s); free(hr); free(role); free(anchor);
  free(beta); free(dnorm); free(wfold); free(a_agg); free(dvec); free(cand_s); free(cand_id);
  return ORC_OK;
}

void orc_dosa_rows(const orc_problem* P, const orc_dosa_params* dp, const int32_t* seeds,
                   const int32_t* rows, int32_t n_rows, int32_t* out_idx, double* out_score,
                   orc_dosa_row_stats* st) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i)
    orc_dosa_row(P, dp, seeds, rows[i], out_idx + (int64_t)i * P->topk,
                 out_score ? out_score + (int64_t)i * P->topk : NULL, st ? st + i : NULL, NULL);
}
