/*
 * sparse_indexer.h - C ABI of the MI355X (gfx950) sparse-attention indexer
 * hot path.
 *
 * Operations, each defined by the page cited at its declaration:
 *   idx_score_topk       lightning-indexer score + per-query top-K
 *   idx_score_topk_witness idx_score_topk then kvwitness_merge, in one pass
 *   idx_score_topk_fused the same from a single kernel (prefill layout)
 *   idx_score_topk_prior the same result on the decode path, selecting only
 *                        among keys above a threshold from recent keys
 *   dosa_prune_topk      the same top-K through DoSA's certified prune
 *   kvwitness_merge      segment-witness covering merge, in place
 *   block_sparse_select  MiniMax-M3 block-sparse block selection
 *   positions_of_blocks  the positions a block selection covers
 *   gather_slots         KV slots of a selection row (flat or paged KV)
 *
 * Conventions shared by every call:
 *  - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; scratch space is passed in as
 *    `workspace` whose size comes from the matching *_workspace() query
 *    (a pure host function).  Passing more workspace than asked is fine.
 *  - Every call is asynchronous on the caller's `stream`.
 *  - Every argument the host can check is checked before any launch; a
 *    refused call writes nothing.  Device-side launch failures come back as
 *    SI_ERR_DEVICE.  No call keeps state between calls; calls are safe from
 *    several threads on different streams.
 *  - Values the host cannot see without a sync (lengths, offsets and
 *    positions held in device memory) are clamped on the device so that no
 *    kernel ever reads or writes out of bounds; out-of-contract values then
 *    give defined but meaningless results.  Inputs are assumed finite.
 *  - Index outputs are row-relative int32, padded with -1.
 *  - Ordering: "top-K" always means the first min(K, n) items under the
 *    total order (score descending, index ascending), -0 == +0; this one
 *    order makes tied ids reproducible everywhere.  A NaN score (outside
 *    the contract) ranks and is reported as -inf; no input bits make a
 *    selection kernel read or write out of bounds.
 */
#ifndef SPARSE_INDEXER_H
#define SPARSE_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SI_OK = 0,
  SI_ERR_INVALID_ARGUMENT = 1,
  /* "Segment Witnesses" page, Refusals: RowsMismatch - the context lengths
   * do not cover every row (here: context_lens is NULL while rows > 0). */
  SI_ERR_ROWS_MISMATCH = 2,
  /* same table: SegmentsOutOfRange - more than 64 segments at the merge */
  SI_ERR_SEGMENTS_OUT_OF_RANGE = 3,
  /* same table: LearnedKeepOutOfRange - the retained prefix is wider than the row */
  SI_ERR_LEARNED_KEEP_OUT_OF_RANGE = 4,
  SI_ERR_UNSUPPORTED_DTYPE = 5,
  SI_ERR_WORKSPACE_TOO_SMALL = 6,
  SI_ERR_DEVICE = 7,
  /* idx_score_topk_noalloc: the problem needs more scratch than the
   * library's fixed array holds (SI_NOALLOC_SCRATCH_BYTES) */
  SI_ERR_SCRATCH_LIMIT = 8
} si_status;

typedef enum { SI_F32 = 0, SI_BF16 = 1, SI_FP8_E4M3FN = 2 } si_dtype;

/* Largest number of witness segments: occupancy travels as one 64-bit mask
 * ("Segment Witnesses" page, Refusals). */
#define SI_MAX_TOPOLOGY_SEGMENTS 64
/* MiniMax-M3's KV block: 128 tokens, also the KV page size (ferrox_core
 * block_sparse.rs, module docs "The block size is an ABI"). */
#define SI_MINIMAX_BLOCK_SIZE 128

/* ------------------------------------------------------------------------ *
 * idx_score_topk
 *
 * DoSA reading notes (notes.kuangjux.top), section 3: the indexer score of
 * key k for a query is  s(k) = sum_h w_h * max(q_h . k, 0)  - all query heads
 * share one index key, weights are signed.  Section 1: the indexer scores
 * every visible key and keeps the top-K.
 *
 *  q       [n_q, H, D], q_dtype SI_F32 or SI_BF16, row-major.
 *  k       [n_k, D], k_dtype SI_F32, SI_BF16 or SI_FP8_E4M3FN (OCP e4m3fn).
 *  k_scale [n_k] f32 per-token scale, required iff k is fp8, else ignored.
 *          The key is k_scale[j] * e4m3fn(k[j, :]); scales must be > 0.
 *  w       f32; weight of (row r, head h) is w[r * w_row_stride + h];
 *          w_row_stride 0 shares one [H] weight vector by all rows.
 *  k_row_offset [n_q] i64 or NULL.  Row r sees keys
 *          k[off_r + j], j in [0, vis_r), off_r = k_row_offset[r] (0 if NULL),
 *          vis_r = clamp(vis_len[r], 0, min(max_vis, n_k - off_r)).
 *          Row-relative index j is what the outputs hold; the query sits at
 *          j = vis_r - 1 ("Segment Witnesses" page, Coordinates contract).
 *  vis_len [n_q] i32.
 *  max_vis host-side upper bound of every vis_r; sizes the workspace.
 *  topk    K >= 1.
 *  out_idx [n_q, K] i32: the top-K of row r (order above), then -1 padding.
 *  out_score [n_q, K] f32 or NULL: their scores, then -inf padding.
 *  q, k must be 16-byte aligned; float outputs 4-byte aligned.
 *  workspace  idx_score_topk_workspace(...) bytes, 256-byte aligned: the
 *          score rows and, for max_vis > 8192, the chunked top-K's
 *          candidate lists.
 * Errors: INVALID_ARGUMENT (null pointer, size <= 0 where one is required,
 * D or H beyond the supported range, misalignment), UNSUPPORTED_DTYPE,
 * WORKSPACE_TOO_SMALL.
 * ------------------------------------------------------------------------ */
si_status idx_score_topk(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                         const float* k_scale, const float* w, int64_t w_row_stride,
                         const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                         int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                         int32_t* out_idx, float* out_score, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
size_t idx_score_topk_workspace(int32_t n_q, int32_t H, int32_t D, int64_t max_vis, int32_t topk);

/* ------------------------------------------------------------------------ *
 * idx_score_topk_noalloc
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * call and result as idx_score_topk (bit for bit), without a workspace
 * argument: the score rows and candidate lists live in a fixed array inside
 * the library, SI_NOALLOC_SCRATCH_BYTES per GPU, allocated when the library
 * is loaded on that GPU and held until the process ends.  The call itself
 * allocates nothing; its first call on a GPU looks the array's address up
 * once (a runtime query, no allocation).
 * Limit: idx_score_topk_workspace(n_q, H, D, max_vis, topk) must be at most
 * SI_NOALLOC_SCRATCH_BYTES (128 MiB: e.g. 4096 queries x 8192 keys, or 128
 * decode rows of up to 131072 keys); a larger problem is refused with
 * SI_ERR_SCRATCH_LIMIT before anything runs.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (several streams, several host threads) race and must be ordered by
 * the caller.  The array keeps the last call's contents; nothing in it needs
 * to start at zero.  The GPU is the device of `stream` (the current device
 * for the null stream).
 * Arguments and other errors as idx_score_topk; SI_ERR_DEVICE also when the
 * array's address cannot be obtained.
 * ------------------------------------------------------------------------ */
#define SI_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
si_status idx_score_topk_noalloc(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                                 const float* k_scale, const float* w, int64_t w_row_stride,
                                 const int64_t* k_row_offset, const int32_t* vis_len,
                                 int32_t n_q, int32_t H, int32_t D, int64_t n_k, int64_t max_vis,
                                 int32_t topk, int32_t* out_idx, float* out_score,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * idx_score_topk_witness
 *
 * idx_score_topk followed by kvwitness_merge on its output rows (the
 * "Segment Witnesses" page, Implementation rule and contracts, applied to
 * the learned top-K rows), with the merge done by the top-K kernel on each
 * row as it is written: out_idx equals idx_score_topk's out_idx after
 * kvwitness_merge(out_idx, n_q, topk, context_lens, num_segments, keep,
 * max_replacements), bit for bit; out_score is idx_score_topk's (the merge
 * changes ids only).  Arguments as the two calls; the merge's refusals are
 * checked first, in its order, then the indexer's.  num_segments == 0 or a
 * budget of 0 gives idx_score_topk's result.  The workspace is
 * idx_score_topk_workspace's.
 * ------------------------------------------------------------------------ */
si_status idx_score_topk_witness(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                                 const float* k_scale, const float* w, int64_t w_row_stride,
                                 const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                                 int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                                 int32_t* out_idx, float* out_score,
                                 const int32_t* context_lens, int32_t num_segments, int32_t keep,
                                 int32_t max_replacements, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * idx_score_topk_fused
 *
 * idx_score_topk_witness computed by ONE kernel for the prefill layout: each
 * workgroup scores its query rows, writes them to the workspace and selects
 * their top-K (then the witness merge) while the rows are still in cache -
 * the score writeback and selection input the DoSA reading notes, section 5,
 * name as costs.  Results equal idx_score_topk_witness's bit for bit (and
 * idx_score_topk's when num_segments or the budget is 0).  On MI355X it is
 * slower than idx_score_topk_witness's two kernels at every prefill size
 * measured (8192 x 8192 H64: 0.55 against 0.51 ms), because a workgroup's
 * selection stalls the MFMA work that would otherwise run on its SIMDs; it
 * is kept for callers that want one launch.
 * Supported: k_row_offset NULL (shared keys), bf16 q and k, H <= 64, D 64 or
 * 128, n_k * D * 2 <= 2 MiB, max_vis <= 8192, topk <= 2048; other shapes ->
 * SI_ERR_UNSUPPORTED_DTYPE.  Arguments, workspace and other errors as
 * idx_score_topk_witness.
 * ------------------------------------------------------------------------ */
si_status idx_score_topk_fused(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                               const float* k_scale, const float* w, int64_t w_row_stride,
                               const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                               int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                               int32_t* out_idx, float* out_score, const int32_t* context_lens,
                               int32_t num_segments, int32_t keep, int32_t max_replacements,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * idx_score_topk_prior
 *
 * The decoding path of the DoSA reading notes, section 1: full FP8 (or bf16)
 * scoring is kept, and a threshold built from recently selected keys cuts
 * the score writeback and the selection work.  The threshold follows the
 * notes' section 2 step 1: tau_r is the K-th largest score among at least K
 * distinct visible keys, here the distinct ids of prior_ids row r in
 * [0, vis_r), scored with every head; with fewer than K of them, tau_r is
 * -inf.  Since those are K keys of the row, the row's K-th largest score is
 * >= tau_r, and only keys with s >= tau_r are written and selected from.
 *
 * Arguments, layout and outputs as idx_score_topk, plus:
 *  prior_ids  [n_q, prior_width] i32, row-relative ids (e.g. the previous
 *          step's out_idx); entries outside [0, vis_r) and repeats are
 *          ignored.  1 <= prior_width <= SI_MAX_PRIOR_WIDTH.
 *  out_tau    [n_q] f32 or NULL: tau_r.
 *  out_survivors [n_q] i32 or NULL: keys with s >= tau_r.
 *  workspace  idx_score_topk_prior_workspace(n_q, max_vis, topk) bytes,
 *          256-byte aligned.
 * out_idx / out_score equal idx_score_topk's bit for bit whatever the prior.
 * Supported: per-row keys (k_row_offset non-NULL), bf16 queries, bf16 or
 * fp8 keys, H <= 64, D 64 or 128; other shapes or dtypes ->
 * UNSUPPORTED_DTYPE.  Other errors as idx_score_topk.
 * ------------------------------------------------------------------------ */
#define SI_MAX_PRIOR_WIDTH 2048
si_status idx_score_topk_prior(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                               const float* k_scale, const float* w, int64_t w_row_stride,
                               const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                               int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                               const int32_t* prior_ids, int32_t prior_width, int32_t* out_idx,
                               float* out_score, float* out_tau, int32_t* out_survivors,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t idx_score_topk_prior_workspace(int32_t n_q, int64_t max_vis, int32_t topk);

/* The two stages of idx_score_topk, for callers that keep the score rows
 * (the notes' section 5 names score writeback and the selection input as
 * costs of their own).
 *
 * idx_score: arguments as idx_score_topk; writes s[r, j] for j < vis_r into
 *   out_scores[r * score_stride + j] (f32, device, score_stride >= max_vis);
 *   entries j >= vis_r are not written.
 * rows_topk: top-K of each row's first vis_r scores (vis_r clamped as in
 *   idx_score_topk from vis_len / k_row_offset / n_k / max_vis), written as
 *   idx_score_topk writes them.  scores rows at r * score_stride.  Rows
 *   longer than 8192 scores (with topk <= 2048) are selected in chunks whose
 *   candidate lists live in the caller's workspace of
 *   rows_topk_workspace(n_rows, max_vis, topk) bytes (0 when not needed;
 *   256-byte aligned); a smaller workspace -> WORKSPACE_TOO_SMALL. */
si_status idx_score(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                    const float* k_scale, const float* w, int64_t w_row_stride,
                    const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q, int32_t H,
                    int32_t D, int64_t n_k, int64_t max_vis, float* out_scores,
                    int64_t score_stride, hipStream_t stream);
si_status rows_topk(const float* scores, int64_t score_stride, const int32_t* vis_len,
                    const int64_t* k_row_offset, int64_t n_k, int64_t max_vis, int32_t n_rows,
                    int32_t topk, int32_t* out_idx, float* out_score, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);
size_t rows_topk_workspace(int32_t n_rows, int64_t max_vis, int32_t topk);

/* ------------------------------------------------------------------------ *
 * dosa_prune_topk
 *
 * DoSA reading notes, section 2: (1) fully score >= K seed keys, take the
 * K-th highest seed score as a fixed threshold tau and keep the seeds'
 * top-K; (2) for every other visible key build a safe upper bound U from the
 * kept heads' exact activations, a single-anchor residual bound for omitted
 * positive heads (section 3.1) and a ReLU-aggregated lower bound of the
 * omitted negative heads' deduction (section 3.2), excluding the key iff
 * U < tau; (3) rescore survivors exactly, drop those below tau, and take the
 * final top-K over the seeds' top-K plus the kept survivors.  Section 4:
 * with no prior, 4 evenly spaced representative queries are fully scored and
 * 12,288 seeds are chosen by occurrence counts in their top-2048 lists;
 * error states trigger an exact recovery.
 *
 * Prefill layout: keys are shared by all rows (no row offsets), q and k are
 * SI_BF16, D is 64 or 128, 1 <= H <= 64, w as in idx_score_topk, row r sees
 * keys [0, vis_r) with vis_r = clamp(vis_len[r], 0, n_k).
 * The result is bit-identical to idx_score_topk on the same device for the
 * same inputs (idx and scores).
 *
 *  params->n_seeds           seeds, topk <= n_seeds <= n_k; 12288 on the page.
 *  params->n_rep_queries     representative rows for the cold prior (1..64),
 *                            row round(i (n_q-1)/(R-1)) for i = 0..R-1.
 *  params->rep_topk          top list length per representative row (1..4096).
 *  params->kept_heads        heads scored exactly in the bound (0..min(31, H)),
 *                            the largest |w_h| * mean max(x_h, 0) over the
 *                            activation sample: 128 seeds evenly spaced in
 *                            seed order, round(i (n_seeds-1)/127) (all seeds
 *                            when fewer; section 4 samples 128 positions of
 *                            the seed region).
 *  params->neg_active_frac   omitted negative heads whose activation
 *                            frequency over that sample is >= this are
 *                            aggregated; the rest are dropped (safe).
 *  params->seed_ids          device [n_seeds] strictly increasing key ids
 *                            visible to every row, or NULL for the cold
 *                            prior (the hook a prior from earlier queries
 *                            would use).
 *  params->survivor_capacity survivors a row may keep (1..8192); a row with
 *                            more takes the exact unpruned path.
 *  params->shared_streams    0: one survivor stream per row.  1: the
 *                            section-4 compaction variant: rows in groups
 *                            of 4 (rows 4g..4g+3); keys passing the bound
 *                            for at least 2 of a group's rows and inside
 *                            its common visible prefix form the group's
 *                            shared stream, rescored once per key tile for
 *                            all 4 rows; the rest go to per-row solo
 *                            streams.  Rows over survivor_capacity take the
 *                            exact path, as with per-row streams, and no
 *                            part in their group's split.  The result is
 *                            the same either way.
 * The workspace (dosa_prune_topk_workspace) holds the seed scores
 * [n_q, n_seeds], survivor lists [n_q, capacity] and, for the exact path,
 * full score rows [n_q, n_k] (f32).
 *  stats (optional, device pointers, each may be NULL): tau [n_q],
 *        n_survivors [n_q] (keys passing the bound; for a row over the
 *        capacity, the count at which its scan stopped, above the
 *        capacity), fallback [n_q] (1 when
 *        the row took the exact path), n_shared [n_q] (those of the row's
 *        survivors its group's shared stream carries; 0 without shared
 *        streams).
 * Rows fall back to the exact path as a whole when fewer than n_seeds keys
 * are visible to every row.
 * Errors: as idx_score_topk, plus INVALID_ARGUMENT for params out of range
 * and for key matrices of 2^31 bytes or more (n_k * D * 2 > INT32_MAX).
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_seeds;
  int32_t n_rep_queries;
  int32_t rep_topk;
  int32_t kept_heads;
  float neg_active_frac;
  const int32_t* seed_ids;
  int32_t survivor_capacity;
  int32_t shared_streams;
} si_dosa_params;

typedef struct {
  float* tau;
  int32_t* n_survivors;
  int32_t* fallback;
  int32_t* n_shared;
} si_dosa_stats;

si_status dosa_prune_topk(const void* q, const void* k, si_dtype dtype, const float* w,
                          int64_t w_row_stride, const int32_t* vis_len, int32_t n_q, int32_t H,
                          int32_t D, int64_t n_k, int32_t topk, const si_dosa_params* params,
                          int32_t* out_idx, float* out_score, const si_dosa_stats* stats,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t dosa_prune_topk_workspace(int32_t n_q, int32_t H, int32_t D, int64_t n_k, int32_t topk,
                                 const si_dosa_params* params);

/* ------------------------------------------------------------------------ *
 * kvwitness_merge  (in place)
 *
 * "Segment Witnesses" page (teerth.dev, Aether-Lang kvwitness), sections
 * Object and Implementation rule and contracts.  For row r with context
 * length L = context_lens[r] and S_eff = min(S, L), segment s < S_eff is
 * [e_s, e_{s+1}) with e_s = ceil(s L / S_eff); an entry x in [0, L) occupies
 * floor(x S_eff / L), an entry x >= L occupies min(floor(x S_eff / L), S - 1),
 * negative entries are padding.  Witnesses e_s of the unoccupied s < S_eff,
 * in ascending s, overwrite slots keep, keep+1, ... up to
 * B = min(max_replacements, topk - keep); the rest are dropped.  Occupancy
 * is read from the whole row before any write.  Rows with L <= 0 are left
 * unchanged.  The serving entry uses keep = topk - S (saturating) and
 * max_replacements = S.
 *
 *  topk_idx     [rows, topk] i32 device, modified in place.
 *  context_lens [rows] i32 device.
 * Check order (a refused call writes nothing): negative rows/topk/keep/
 * max_replacements -> INVALID_ARGUMENT; context_lens NULL with rows > 0 ->
 * ROWS_MISMATCH; topk_idx NULL with rows, topk > 0 -> INVALID_ARGUMENT;
 * num_segments < 0 or > 64 -> SEGMENTS_OUT_OF_RANGE; keep > topk ->
 * LEARNED_KEEP_OUT_OF_RANGE.  Then num_segments == 0 (the off switch),
 * B == 0 or rows == 0 return SI_OK without touching anything.
 * ------------------------------------------------------------------------ */
si_status kvwitness_merge(int32_t* topk_idx, int32_t rows, int32_t topk,
                          const int32_t* context_lens, int32_t num_segments, int32_t keep,
                          int32_t max_replacements, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * block_sparse_select
 *
 * ferrox_core block_sparse.rs (docs.rs, ferrox-core 0.14.0): module docs
 * "Four rules", the public selection entry's doc comment and the per-head
 * selection's comments on scoring and ties.  For query i at position
 * p = query_pos[i]: n_blocks = min(p / block_size + 1, ceil(n_pos /
 * block_size)) (0 when p < 0).  Per KV head h independently: the first
 * min(init_blocks, n) and the last min(local_blocks, n) blocks are forced;
 * budget = max(top_blocks, #forced); if the forced set already fills the
 * budget or every block, it is the selection; otherwise every other block is
 * scored by the MAX over its positions [b*bs, min((b+1)*bs, n_pos, p+1)) of
 * the f32 dot of index_q[i, h] and index_k[pos] - summed in index order,
 * each product rounded to f32 before it is added, starting from +0 - and
 * the best budget - #forced by (score desc, block asc) join the forced
 * ones.  The selection is written ascending.
 *
 *  index_q    [n_q, n_kv_heads, D] f32.   index_k [n_pos, D] f32.
 *  query_pos  [n_q] i64.
 *  out_blocks [n_q, n_kv_heads, out_width] i32, ascending, then -1.
 *  out_count  [n_q, n_kv_heads] i32 (may be NULL).
 *  out_width  >= max(top_blocks, init_blocks + local_blocks).
 * Errors: INVALID_ARGUMENT (null pointers, block_size <= 0, negative
 * counts, out_width too small, D out of range), WORKSPACE_TOO_SMALL.
 * ------------------------------------------------------------------------ */
si_status block_sparse_select(const float* index_q, const float* index_k,
                              const int64_t* query_pos, int32_t n_q, int32_t n_kv_heads,
                              int32_t D, int64_t n_pos, int32_t block_size, int32_t top_blocks,
                              int32_t init_blocks, int32_t local_blocks, int32_t* out_blocks,
                              int32_t out_width, int32_t* out_count, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);
size_t block_sparse_select_workspace(int32_t n_q, int32_t n_kv_heads, int64_t n_pos,
                                     int32_t block_size);

/* ------------------------------------------------------------------------ *
 * positions_of_blocks
 *
 * ferrox_core block_sparse.rs (docs.rs, ferrox-core 0.14.0), the
 * positions helper's doc comment: the positions a block list covers,
 * ascending and
 * deduplicated, each block b covering [b*bs, min((b+1)*bs, n_pos, p+1))
 * for the query at p = query_pos[i] (nothing when p < 0).  Negative entries
 * are padding and cover nothing; the list may be in any order and repeat
 * blocks.
 *
 *  blocks    [n_q, n_kv_heads, width] i32 (e.g. block_sparse_select's
 *            out_blocks), 0 <= width <= 4096.
 *  query_pos [n_q] i64, shared by the query's KV heads.
 *  out_pos   [n_q, n_kv_heads, out_width] i32: the covered positions, then
 *            -1.  out_width >= min(width * block_size, n_pos), so every
 *            covered position fits.
 *  out_count [n_q, n_kv_heads] i32 (may be NULL): positions covered.
 * Errors: INVALID_ARGUMENT (negative counts, block_size < 1, width > 4096,
 * n_pos outside [0, 2^31 - 1], out_width too small, null pointers).
 * ------------------------------------------------------------------------ */
si_status positions_of_blocks(const int32_t* blocks, int32_t n_q, int32_t n_kv_heads,
                              int32_t width, const int64_t* query_pos, int64_t n_pos,
                              int32_t block_size, int32_t* out_pos, int32_t out_width,
                              int32_t* out_count, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * gather_slots
 *
 * Where the attention that consumes a selection row reads each entry.  The
 * "Segment Witnesses" page (Implementation rule and contracts: Coordinates)
 * makes the entries of a (witness-merged) top-K row row-relative offsets:
 * row r's tokens are [0, L_r), -1 is padding, and a learned entry >= L_r
 * passes through the merge without naming a token of the row.  Entry x of
 * row r is gathered iff 0 <= x < L_r, at
 *   row_start[r] + x                                    (flat KV buffer), or
 *   page_table[r][x / page_size] * page_size + x % page_size   (paged KV; the
 *   block-sparse page makes its 128-token block the KV page),
 * and every other entry, a page index >= pages_per_row and a negative page
 * id give -1.  The row's order is kept.
 *
 *  idx        [rows, width] i32 (e.g. kvwitness_merge's output rows, or
 *             positions_of_blocks' lists with L_r = n_pos).
 *  lens       [rows] i32: L_r.
 *  row_start  [rows] i64, or NULL when page_table is given (exactly one).
 *  page_table [rows, pages_per_row] i32 physical page ids.
 *  out_slots  [rows, width] i64.
 * Errors: INVALID_ARGUMENT (negative counts, both or neither mapping,
 * page_size or pages_per_row < 1 with a page table, width > 2^25, null
 * pointers).
 * ------------------------------------------------------------------------ */
si_status gather_slots(const int32_t* idx, int32_t rows, int32_t width, const int32_t* lens,
                       const int64_t* row_start, const int32_t* page_table,
                       int32_t pages_per_row, int32_t page_size, int64_t* out_slots,
                       hipStream_t stream);

const char* si_status_string(si_status status);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_INDEXER_H */
