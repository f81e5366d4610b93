/*
 * Plain CPU oracle for the sparse-attention indexer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this.  It shares no source, header,
 * table or helper with the HIP library; both sides only read the same
 * synthetic input bytes.
 *
 * Floating point: indexer scores are accumulated in double from inputs that
 * are exactly representable in double (f32, bf16, OCP fp8 e4m3fn x f32
 * scale), so a score is the real-valued definition up to ~1e-15 relative.
 * Block-sparse dots follow the page's f32 definition exactly (sequential,
 * product rounded to f32, then added; the file is built with
 * -ffp-contract=off so no fused multiply-add can appear).
 *
 * Status codes returned by the witness merge mirror the refusal kinds of the
 * "Segment Witnesses" page, section "Refusals".
 */
#ifndef SPARSE_INDEXER_ORACLE_H
#define SPARSE_INDEXER_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3FN = 2 };

enum {
  ORC_OK = 0,
  ORC_INVALID_ARGUMENT = 1,
  ORC_ROWS_MISMATCH = 2,
  ORC_SEGMENTS_OUT_OF_RANGE = 3,
  ORC_KEEP_OUT_OF_RANGE = 4,
  ORC_NOT_ENOUGH_KEYS = 5
};

/* One indexer problem: queries q[n_q,H,D], keys k[n_k,D] (fp8 keys carry a
 * per-token scale), weights w[r*w_row_stride + h], row r sees keys
 * [off_r, off_r + vis_r) where off_r = k_row_offset ? k_row_offset[r] : 0 and
 * vis_r = clamp(vis_len[r], 0, min(max_vis, n_k - off_r)). */
typedef struct {
  const void* q;
  int32_t q_dtype;
  const void* k;
  int32_t k_dtype;
  const float* k_scale;
  const float* w;
  int64_t w_row_stride;
  const int64_t* k_row_offset;
  const int32_t* vis_len;
  int32_t n_q, H, D;
  int64_t n_k, max_vis;
  int32_t topk;
} orc_problem;

double orc_decode(const void* p, int32_t dtype, int64_t i);
double orc_e4m3fn_to_double(uint8_t b);
int64_t orc_visible(const orc_problem* P, int32_t r);

/* Score of every visible key of row r: s[j], plus the tolerance scales
 * m[j] = sum_h |w_h| max(0, x_h) and n[j] = sum_h |w_h| |q_h| |k_j|.
 * Any of s/m/n may be NULL.  Returns the visible count. */
int64_t orc_score_row(const orc_problem* P, int32_t r, double* s, double* m, double* n);

/* Top-K of n scored items by (score desc, id asc); ids NULL means id = position.
 * Writes min(K, n) entries then pads -1 / -inf.  Returns min(K, n). */
int32_t orc_topk(const double* s, const int32_t* ids, int64_t n, int32_t K,
                 int32_t* out_idx, double* out_score);

/* Rows rows[0..n_rows) of the full indexer: top-K ids and scores, and
 * optionally the full score/m/n rows (row i at i*row_stride). */
void orc_idx_score_topk_rows(const orc_problem* P, const int32_t* rows, int32_t n_rows,
                             int32_t* out_idx, double* out_score, double* s_rows,
                             double* m_rows, double* n_rows_out, int64_t row_stride);

/* ---- Segment witnesses ---- */
int64_t orc_segment_of(int64_t token, int64_t context_len, int64_t num_segments);
int64_t orc_segment_edge(int64_t s, int64_t L, int64_t S_eff);
int64_t orc_occupied_segment(int64_t x, int64_t L, int64_t S);
int32_t orc_witness_indices(const int32_t* learned, int32_t rows, int32_t topk,
                            const int32_t* context_lens, int32_t num_segments, int32_t* out);
int32_t orc_kvwitness_merge(int32_t* topk_idx, int32_t rows, int32_t topk,
                            const int32_t* context_lens, int32_t num_segments, int32_t keep,
                            int32_t max_replacements);
double orc_segment_coverage(const int32_t* cand, int32_t n, int64_t L, int64_t num_segments);

/* ---- Block-sparse selection ---- */
float orc_block_dot(const float* a, const float* b, int32_t D);
int64_t orc_causal_blocks(int64_t query_pos, int64_t block_size);
int32_t orc_block_select_query(const float* q /*[H,D]*/, const float* k /*[n_pos,D]*/,
                               int64_t query_pos, int32_t H, int32_t D, int64_t n_pos,
                               int32_t block_size, int32_t top_blocks, int32_t init_blocks,
                               int32_t local_blocks, int32_t* out /*[H,width]*/, int32_t width,
                               int32_t* counts /*[H]*/, float* block_scores /*[H,n_blocks] or NULL*/);
void orc_block_select_rows(const float* q /*[n_q,H,D]*/, const float* k, const int64_t* query_pos,
                           const int32_t* rows, int32_t n_rows, int32_t H, int32_t D,
                           int64_t n_pos, int32_t block_size, int32_t top_blocks,
                           int32_t init_blocks, int32_t local_blocks, int32_t* out,
                           int32_t width, int32_t* counts);
int64_t orc_positions_of_blocks(const int32_t* blocks, int32_t n_blocks_sel, int64_t query_pos,
                                int64_t n_pos, int32_t block_size, int64_t* out);
void orc_positions_of_block_rows(const int32_t* blocks, int32_t n_q, int32_t n_heads,
                                 int32_t width, const int64_t* query_pos, int64_t n_pos,
                                 int32_t block_size, int32_t* out, int64_t out_width,
                                 int32_t* count);
void orc_gather_slots(const int32_t* idx, int32_t rows, int32_t width, const int32_t* lens,
                      const int64_t* row_start, const int32_t* page_table, int32_t pages_per_row,
                      int32_t page_size, int64_t* out);

/* ---- DoSA certified prune ---- */
typedef struct {
  int32_t n_seeds, n_rep_queries, rep_topk, kept_heads;
  double neg_active_frac;
  int64_t survivor_capacity;
} orc_dosa_params;

typedef struct {
  double tau;
  int32_t n_kept_heads, n_pos_omitted, n_neg_aggregated, n_neg_dropped;
  int64_t n_scanned, n_survivors, n_kept_survivors;
  int32_t fallback;
  int64_t head_dots;
  double R;
} orc_dosa_row_stats;

/* Optional per-row diagnostics; every pointer may be NULL. */
typedef struct {
  int32_t* head_role;  /* [H]: 1 kept, 2 omitted positive, 3 aggregated negative,
                          4 dropped negative, 0 zero weight */
  int32_t* anchor;     /* [H] kept anchor head of an omitted positive head, else -1 */
  double* beta;        /* [H] */
  double* dnorm;       /* [H] |d_h| */
  double* wfold;       /* [H] folded weight of kept heads, 0 elsewhere */
  double* act;         /* [H] activation frequency over the seeds */
  double* a_agg;       /* [D] aggregated negative query */
  double* pos_part;    /* [vis] per key: sum_J w'_j max(0,x_j) + R |k|  (NaN for seeds) */
  double* neg_part;    /* [vis] per key: max(0, a_A . k)              (NaN for seeds) */
  double* U;           /* [vis] per key: certified upper bound used    (NaN for seeds) */
} orc_dosa_diag;

int32_t orc_dosa_common_prefix(const orc_problem* P);
int32_t orc_dosa_rep_row(int32_t i, int32_t n_rep, int32_t n_q);
int32_t orc_dosa_seeds(const orc_problem* P, const orc_dosa_params* dp, int32_t* seeds,
                       int32_t* counts /*[c] or NULL*/);
int32_t orc_dosa_row(const orc_problem* P, const orc_dosa_params* dp, const int32_t* seeds,
                     int32_t r, int32_t* out_idx, double* out_score, orc_dosa_row_stats* st,
                     const orc_dosa_diag* dg);
void orc_dosa_rows(const orc_problem* P, const orc_dosa_params* dp, const int32_t* seeds,
                   const int32_t* rows, int32_t n_rows, int32_t* out_idx, double* out_score,
                   orc_dosa_row_stats* st);
int64_t orc_dosa_head_dots(int64_t n_seeds, int64_t n_scanned, int64_t filter_dots_per_key,
                           int64_t n_survivors, int32_t H);

int32_t orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
