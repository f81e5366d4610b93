// C-ABI entry points: host-side validation (before any HIP call), workspace
// carving and launches on the caller's stream.  See include/sparse_indexer.h.
#include <string.h>

#include <mutex>

#include "si_internal.hpp"

// The allocation-free entry point's scratch: the score rows and candidate
// lists that idx_score_topk keeps in the caller's workspace.  One copy per
// GPU, held from the library's load on that GPU until the process ends.
// Host code never uses this name as an address: it takes the device
// address from hipGetSymbolAddress (scratch_on_device below).
static __device__ __align__(256) unsigned char scratch[SI_NOALLOC_SCRATCH_BYTES];

namespace si {
hipError_t launch_block_select(const float* q, const float* k, const int64_t* qpos, int32_t n_q,
                               int32_t H, int32_t D, int64_t n_pos, int32_t bs, int32_t top,
                               int32_t init, int32_t local, int32_t* out, int32_t width,
                               int32_t* count, float* ws, hipStream_t st);

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
static inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// Shapes the generic (non-MFMA) score path can hold.
static bool generic_shape_ok(int32_t H, int32_t D) {
  return H >= 1 && H <= 1024 && D >= 1 && (int64_t)H * D <= 8192;
}

static size_t score_ws_bytes(int32_t n_q, int64_t max_vis) {
  if (n_q <= 0 || max_vis <= 0) return 0;
  return align_up((size_t)n_q * (size_t)max_vis * sizeof(float), 256);
}
}  // namespace si

using namespace si;

extern "C" {

const char* si_status_string(si_status s) {
  switch (s) {
    case SI_OK: return "ok";
    case SI_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SI_ERR_ROWS_MISMATCH: return "context lengths do not cover every row";
    case SI_ERR_SEGMENTS_OUT_OF_RANGE: return "num_segments out of range (0..64)";
    case SI_ERR_LEARNED_KEEP_OUT_OF_RANGE: return "keep exceeds the row width";
    case SI_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case SI_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SI_ERR_DEVICE: return "device error";
    case SI_ERR_SCRATCH_LIMIT:
      return "problem needs more than the allocation-free entry point's fixed scratch";
  }
  return "unknown status";
}

size_t rows_topk_workspace(int32_t n_rows, int64_t max_vis, int32_t topk) {
  if (n_rows <= 0 || max_vis <= 0 || topk < 1) return 0;
  return topk_workspace_bytes(n_rows, max_vis, topk);
}

// idx_score_topk's workspace: the score rows, then (256-byte aligned) the
// candidate lists of the chunked top-K for long rows
size_t idx_score_topk_workspace(int32_t n_q, int32_t H, int32_t D, int64_t max_vis, int32_t topk) {
  (void)H;
  (void)D;
  const size_t s = (score_ws_bytes(n_q, max_vis) + 255) & ~(size_t)255;
  return s + rows_topk_workspace(n_q, max_vis, topk);
}

// Checks shared by idx_score and idx_score_topk; fills `sa` (scores unset).
static si_status check_score_args(const void* q, si_dtype q_dtype, const void* k,
                                  si_dtype k_dtype, const float* k_scale, const float* w,
                                  int64_t w_row_stride, const int64_t* k_row_offset,
                                  const int32_t* vis_len, int32_t n_q, int32_t H, int32_t D,
                                  int64_t n_k, int64_t max_vis, ScoreArgs* sa) {
  if (n_q < 0 || H < 1 || D < 1 || n_k < 0 || max_vis < 0 || w_row_stride < 0)
    return SI_ERR_INVALID_ARGUMENT;
  if (q_dtype != SI_F32 && q_dtype != SI_BF16) return SI_ERR_UNSUPPORTED_DTYPE;
  if (k_dtype != SI_F32 && k_dtype != SI_BF16 && k_dtype != SI_FP8_E4M3FN)
    return SI_ERR_UNSUPPORTED_DTYPE;
  if (max_vis > INT32_MAX) return SI_ERR_INVALID_ARGUMENT;  // row-relative ids are int32
  sa->q = q; sa->q_dtype = q_dtype; sa->k = k; sa->k_dtype = k_dtype; sa->k_scale = k_scale;
  sa->w = w; sa->w_row_stride = w_row_stride; sa->k_row_offset = k_row_offset;
  sa->vis_len = vis_len; sa->n_q = n_q; sa->H = H; sa->D = D; sa->n_k = n_k;
  sa->max_vis = max_vis; sa->scores = nullptr; sa->score_stride = max_vis;
  if (!score_mfma_supported(*sa) && !generic_shape_ok(H, D)) return SI_ERR_INVALID_ARGUMENT;
  if (n_q == 0) return SI_OK;
  if (!q || !k || !w || !vis_len) return SI_ERR_INVALID_ARGUMENT;
  if (k_dtype == SI_FP8_E4M3FN && !k_scale) return SI_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned4(w)) return SI_ERR_INVALID_ARGUMENT;
  return SI_OK;
}

si_status idx_score(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                    const float* k_scale, const float* w, int64_t w_row_stride,
                    const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q, int32_t H,
                    int32_t D, int64_t n_k, int64_t max_vis, float* out_scores,
                    int64_t score_stride, hipStream_t stream) {
  ScoreArgs sa;
  si_status s = check_score_args(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset,
                                 vis_len, n_q, H, D, n_k, max_vis, &sa);
  if (s != SI_OK || n_q == 0) return s;
  if (!out_scores || !aligned4(out_scores) || score_stride < max_vis)
    return SI_ERR_INVALID_ARGUMENT;
  sa.scores = out_scores;
  sa.score_stride = score_stride;
  return launch_score(sa, stream) == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

si_status rows_topk(const float* scores, int64_t score_stride, const int32_t* vis_len,
                    const int64_t* k_row_offset, int64_t n_k, int64_t max_vis, int32_t n_rows,
                    int32_t topk, int32_t* out_idx, float* out_score, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (n_rows < 0 || n_k < 0 || max_vis < 0 || max_vis > INT32_MAX || topk < 1 ||
      topk > kMaxTopk || score_stride < max_vis)
    return SI_ERR_INVALID_ARGUMENT;
  if (n_rows == 0) return SI_OK;
  if ((max_vis > 0 && !scores) || !vis_len || !out_idx || !aligned4(out_idx) ||
      (out_score && !aligned4(out_score)) || (scores && !aligned4(scores)))
    return SI_ERR_INVALID_ARGUMENT;
  const size_t need = rows_topk_workspace(n_rows, max_vis, topk);
  if (need && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return SI_ERR_WORKSPACE_TOO_SMALL;
  TopkArgs ta;
  ta.scores = scores; ta.stride = score_stride; ta.vis_len = vis_len;
  ta.k_row_offset = k_row_offset; ta.n_k = n_k; ta.max_vis = max_vis; ta.n_rows = n_rows;
  ta.K = topk; ta.out_idx = out_idx; ta.out_score = out_score; ta.id_map = nullptr;
  ta.workspace = workspace; ta.workspace_bytes = workspace_bytes;
  return launch_topk(ta, stream) == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

// Validates an idx_score_topk call and fills the score and top-K stage
// arguments (the workspace holds the score rows, then the candidate lists);
// *done is set when there is nothing to launch (n_q == 0).
static si_status prepare_score_topk(const void* q, si_dtype q_dtype, const void* k,
                                    si_dtype k_dtype, const float* k_scale, const float* w,
                                    int64_t w_row_stride, const int64_t* k_row_offset,
                                    const int32_t* vis_len, int32_t n_q, int32_t H, int32_t D,
                                    int64_t n_k, int64_t max_vis, int32_t topk, int32_t* out_idx,
                                    float* out_score, void* workspace, size_t workspace_bytes,
                                    ScoreArgs* sa, TopkArgs* ta, bool* done) {
  *done = false;
  si_status s = check_score_args(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset,
                                 vis_len, n_q, H, D, n_k, max_vis, sa);
  if (s != SI_OK) return s;
  if (topk < 1 || topk > kMaxTopk) return SI_ERR_INVALID_ARGUMENT;
  if (n_q == 0) {
    *done = true;
    return SI_OK;
  }
  if (!out_idx || !aligned4(out_idx) || (out_score && !aligned4(out_score)))
    return SI_ERR_INVALID_ARGUMENT;
  const size_t need = idx_score_topk_workspace(n_q, H, D, max_vis, topk);
  if (need && (!workspace || workspace_bytes < need ||
               (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return SI_ERR_WORKSPACE_TOO_SMALL;
  sa->scores = reinterpret_cast<float*>(workspace);
  const size_t cand_off = (score_ws_bytes(n_q, max_vis) + 255) & ~(size_t)255;
  TopkArgs& t = *ta;
  t.scores = sa->scores; t.stride = max_vis; t.vis_len = vis_len; t.k_row_offset = k_row_offset;
  t.n_k = n_k; t.max_vis = max_vis; t.n_rows = n_q; t.K = topk; t.out_idx = out_idx;
  t.out_score = out_score; t.id_map = nullptr;
  t.workspace = static_cast<unsigned char*>(workspace) + cand_off;
  t.workspace_bytes = workspace_bytes - cand_off;
  return SI_OK;
}

// The score kernel, then the top-K kernel (which also merges witnesses when
// ta.wit_lens is set).
static si_status run_score_topk(const ScoreArgs& sa, const TopkArgs& ta, hipStream_t stream) {
  hipError_t e = launch_score(sa, stream);
  if (e == hipSuccess) e = launch_topk(ta, stream);
  return e == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

si_status idx_score_topk(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                         const float* k_scale, const float* w, int64_t w_row_stride,
                         const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                         int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                         int32_t* out_idx, float* out_score, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  ScoreArgs sa;
  TopkArgs ta;
  bool done;
  const si_status s = prepare_score_topk(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride,
                                         k_row_offset, vis_len, n_q, H, D, n_k, max_vis, topk,
                                         out_idx, out_score, workspace, workspace_bytes, &sa, &ta,
                                         &done);
  if (s != SI_OK || done) return s;
  return run_score_topk(sa, ta, stream);
}

// The witness merge's refusals, in kvwitness_merge's order (a refused call
// writes nothing); *B gets the merge budget min(max_replacements, topk -
// keep).
static si_status check_witness_args(int32_t n_q, int32_t topk, const int32_t* out_idx,
                                    const int32_t* context_lens, int32_t num_segments,
                                    int32_t keep, int32_t max_replacements, int32_t* B) {
  if (n_q < 0 || topk < 0 || keep < 0 || max_replacements < 0) return SI_ERR_INVALID_ARGUMENT;
  if (n_q > 0 && !context_lens) return SI_ERR_ROWS_MISMATCH;
  if (n_q > 0 && topk > 0 && !out_idx) return SI_ERR_INVALID_ARGUMENT;
  if (num_segments < 0 || num_segments > SI_MAX_TOPOLOGY_SEGMENTS)
    return SI_ERR_SEGMENTS_OUT_OF_RANGE;
  if (keep > topk) return SI_ERR_LEARNED_KEEP_OUT_OF_RANGE;
  *B = max_replacements < topk - keep ? max_replacements : topk - keep;
  if (n_q > 0 && num_segments > 0 && *B > 0 && !aligned4(context_lens))
    return SI_ERR_INVALID_ARGUMENT;
  return SI_OK;
}

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream), looked up once per device with that device current
// and kept; nullptr on failure.
static void* scratch_on_device(hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return nullptr;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

si_status idx_score_topk_noalloc(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                                 const float* k_scale, const float* w, int64_t w_row_stride,
                                 const int64_t* k_row_offset, const int32_t* vis_len,
                                 int32_t n_q, int32_t H, int32_t D, int64_t n_k, int64_t max_vis,
                                 int32_t topk, int32_t* out_idx, float* out_score,
                                 hipStream_t stream) {
  // every host-side check first (as idx_score_topk's), then the size limit;
  // only then the one runtime query (no allocation: the array exists since
  // the library's code object was loaded on the device)
  ScoreArgs sa;
  si_status s = check_score_args(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset,
                                 vis_len, n_q, H, D, n_k, max_vis, &sa);
  if (s != SI_OK) return s;
  if (topk < 1 || topk > kMaxTopk) return SI_ERR_INVALID_ARGUMENT;
  if (n_q == 0) return SI_OK;
  if (!out_idx || !aligned4(out_idx) || (out_score && !aligned4(out_score)))
    return SI_ERR_INVALID_ARGUMENT;
  const size_t need = idx_score_topk_workspace(n_q, H, D, max_vis, topk);
  if (need > SI_NOALLOC_SCRATCH_BYTES) return SI_ERR_SCRATCH_LIMIT;
  void* ws = scratch_on_device(stream);
  if (ws == nullptr) return SI_ERR_DEVICE;
  return idx_score_topk(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset, vis_len,
                        n_q, H, D, n_k, max_vis, topk, out_idx, out_score, ws,
                        SI_NOALLOC_SCRATCH_BYTES, stream);
}

si_status idx_score_topk_witness(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                                 const float* k_scale, const float* w, int64_t w_row_stride,
                                 const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                                 int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                                 int32_t* out_idx, float* out_score,
                                 const int32_t* context_lens, int32_t num_segments, int32_t keep,
                                 int32_t max_replacements, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  // the merge's refusals first, then the indexer's
  int32_t B;
  si_status s = check_witness_args(n_q, topk, out_idx, context_lens, num_segments, keep,
                                   max_replacements, &B);
  if (s != SI_OK) return s;
  ScoreArgs sa;
  TopkArgs ta;
  bool done;
  s = prepare_score_topk(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset, vis_len,
                         n_q, H, D, n_k, max_vis, topk, out_idx, out_score, workspace,
                         workspace_bytes, &sa, &ta, &done);
  if (s != SI_OK || done) return s;
  if (num_segments > 0 && B > 0) {
    ta.wit_lens = context_lens; ta.wit_S = num_segments; ta.wit_keep = keep; ta.wit_B = B;
  }
  return run_score_topk(sa, ta, stream);
}

si_status idx_score_topk_fused(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                               const float* k_scale, const float* w, int64_t w_row_stride,
                               const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                               int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                               int32_t* out_idx, float* out_score, const int32_t* context_lens,
                               int32_t num_segments, int32_t keep, int32_t max_replacements,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int32_t B;
  si_status s = check_witness_args(n_q, topk, out_idx, context_lens, num_segments, keep,
                                   max_replacements, &B);
  if (s != SI_OK) return s;
  ScoreArgs sa;
  TopkArgs ta;
  bool done;
  s = prepare_score_topk(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset, vis_len,
                         n_q, H, D, n_k, max_vis, topk, out_idx, out_score, workspace,
                         workspace_bytes, &sa, &ta, &done);
  if (s != SI_OK) return s;
  if (!score_topk_fused_supported(sa, topk)) return SI_ERR_UNSUPPORTED_DTYPE;
  if (done) return SI_OK;
  if (num_segments > 0 && B > 0) {
    ta.wit_lens = context_lens; ta.wit_S = num_segments; ta.wit_keep = keep; ta.wit_B = B;
  }
  return launch_score_topk_fused(sa, ta, stream) == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

size_t idx_score_topk_prior_workspace(int32_t n_q, int64_t max_vis, int32_t topk) {
  if (n_q <= 0 || max_vis <= 0 || max_vis > INT32_MAX || topk < 1 || topk > kMaxTopk) return 0;
  return prior_workspace_bytes(n_q, max_vis, topk);
}

si_status idx_score_topk_prior(const void* q, si_dtype q_dtype, const void* k, si_dtype k_dtype,
                               const float* k_scale, const float* w, int64_t w_row_stride,
                               const int64_t* k_row_offset, const int32_t* vis_len, int32_t n_q,
                               int32_t H, int32_t D, int64_t n_k, int64_t max_vis, int32_t topk,
                               const int32_t* prior_ids, int32_t prior_width, int32_t* out_idx,
                               float* out_score, float* out_tau, int32_t* out_survivors,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ScoreArgs sa;
  si_status s = check_score_args(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset,
                                 vis_len, n_q, H, D, n_k, max_vis, &sa);
  if (s != SI_OK) return s;
  if (topk < 1 || topk > kMaxTopk || prior_width < 1 || prior_width > SI_MAX_PRIOR_WIDTH)
    return SI_ERR_INVALID_ARGUMENT;
  // the decode layout on the MFMA path: per-row keys, bf16 queries
  if (q_dtype != SI_BF16 || k_dtype == SI_F32 || !score_mfma_supported(sa))
    return SI_ERR_UNSUPPORTED_DTYPE;
  if (n_q == 0) return SI_OK;
  if (!k_row_offset || !prior_ids || !out_idx || !aligned4(out_idx) ||
      (out_score && !aligned4(out_score)) || (out_tau && !aligned4(out_tau)) ||
      (out_survivors && !aligned4(out_survivors)) || !aligned4(prior_ids))
    return SI_ERR_INVALID_ARGUMENT;
  if (max_vis == 0) {  // nothing visible: the plain path writes the padding
    return idx_score_topk(q, q_dtype, k, k_dtype, k_scale, w, w_row_stride, k_row_offset,
                          vis_len, n_q, H, D, n_k, max_vis, topk, out_idx, out_score, workspace,
                          workspace_bytes, stream);
  }
  const size_t need = idx_score_topk_prior_workspace(n_q, max_vis, topk);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return SI_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = launch_prior_topk(sa, prior_ids, prior_width, topk, out_idx, out_score, out_tau,
                                   out_survivors, workspace, stream);
  return e == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

si_status kvwitness_merge(int32_t* topk_idx, int32_t rows, int32_t topk,
                          const int32_t* context_lens, int32_t num_segments, int32_t keep,
                          int32_t max_replacements, hipStream_t stream) {
  if (rows < 0 || topk < 0 || keep < 0 || max_replacements < 0) return SI_ERR_INVALID_ARGUMENT;
  if (rows > 0 && !context_lens) return SI_ERR_ROWS_MISMATCH;
  if (rows > 0 && topk > 0 && !topk_idx) return SI_ERR_INVALID_ARGUMENT;
  if (num_segments < 0 || num_segments > SI_MAX_TOPOLOGY_SEGMENTS)
    return SI_ERR_SEGMENTS_OUT_OF_RANGE;
  if (keep > topk) return SI_ERR_LEARNED_KEEP_OUT_OF_RANGE;
  const int32_t B = max_replacements < topk - keep ? max_replacements : topk - keep;
  if (num_segments == 0 || B == 0 || rows == 0) return SI_OK;
  if (!aligned4(topk_idx) || !aligned4(context_lens)) return SI_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_witness(topk_idx, rows, topk, context_lens, num_segments, keep, B, stream);
  return e == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

si_status block_sparse_select(const float* index_q, const float* index_k,
                              const int64_t* query_pos, int32_t n_q, int32_t n_kv_heads,
                              int32_t D, int64_t n_pos, int32_t block_size, int32_t top_blocks,
                              int32_t init_blocks, int32_t local_blocks, int32_t* out_blocks,
                              int32_t out_width, int32_t* out_count, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (n_q < 0 || n_kv_heads < 1 || D < 1 || D > 65536 || n_pos < 0 || block_size < 1 ||
      top_blocks < 0 || init_blocks < 0 || local_blocks < 0)
    return SI_ERR_INVALID_ARGUMENT;
  const int64_t need_w = top_blocks > (int64_t)init_blocks + local_blocks
                             ? top_blocks
                             : (int64_t)init_blocks + local_blocks;
  if (out_width < need_w || out_width < 1 || out_width > kMaxTopk) return SI_ERR_INVALID_ARGUMENT;
  const int64_t max_blocks = (n_pos + block_size - 1) / block_size;
  if (max_blocks > INT32_MAX) return SI_ERR_INVALID_ARGUMENT;
  if (n_q == 0) return SI_OK;
  if (!index_q || (!index_k && n_pos > 0) || !query_pos || !out_blocks)
    return SI_ERR_INVALID_ARGUMENT;
  if ((int64_t)n_q * n_kv_heads > INT32_MAX) return SI_ERR_INVALID_ARGUMENT;
  const int64_t qt = n_kv_heads >= 32 ? 1 : 32 / n_kv_heads;
  if (((n_q + qt - 1) / qt) * max_blocks > INT32_MAX) return SI_ERR_INVALID_ARGUMENT;
  const size_t need = block_sparse_select_workspace(n_q, n_kv_heads, n_pos, block_size);
  if (need && (!workspace || workspace_bytes < need || !aligned4(workspace)))
    return SI_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = launch_block_select(index_q, index_k, query_pos, n_q, n_kv_heads, D, n_pos,
                                     block_size, top_blocks, init_blocks, local_blocks, out_blocks,
                                     out_width, out_count, reinterpret_cast<float*>(workspace),
                                     stream);
  return e == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

si_status positions_of_blocks(const int32_t* blocks, int32_t n_q, int32_t n_kv_heads,
                              int32_t width, const int64_t* query_pos, int64_t n_pos,
                              int32_t block_size, int32_t* out_pos, int32_t out_width,
                              int32_t* out_count, hipStream_t stream) {
  if (n_q < 0 || n_kv_heads < 0 || width < 0 || width > kMaxTopk || block_size < 1 ||
      n_pos < 0 || n_pos > INT32_MAX || out_width < 0)
    return SI_ERR_INVALID_ARGUMENT;
  const int64_t most = (int64_t)width * block_size < n_pos ? (int64_t)width * block_size : n_pos;
  if (out_width < most) return SI_ERR_INVALID_ARGUMENT;
  if ((int64_t)n_q * n_kv_heads > INT32_MAX) return SI_ERR_INVALID_ARGUMENT;
  if (n_q == 0 || n_kv_heads == 0) return SI_OK;
  if (!query_pos || (out_width > 0 && !out_pos) || (width > 0 && !blocks))
    return SI_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_block_positions(blocks, n_q, n_kv_heads, width, query_pos, n_pos,
                                        block_size, out_pos, out_width, out_count, stream);
  return e == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

si_status gather_slots(const int32_t* idx, int32_t rows, int32_t width, const int32_t* lens,
                       const int64_t* row_start, const int32_t* page_table,
                       int32_t pages_per_row, int32_t page_size, int64_t* out_slots,
                       hipStream_t stream) {
  if (rows < 0 || width < 0 || width > (1 << 25)) return SI_ERR_INVALID_ARGUMENT;  // grid y <= 32768
  if ((row_start == nullptr) == (page_table == nullptr)) return SI_ERR_INVALID_ARGUMENT;
  if (page_table && (page_size < 1 || pages_per_row < 1)) return SI_ERR_INVALID_ARGUMENT;
  if (rows == 0 || width == 0) return SI_OK;
  if (!idx || !lens || !out_slots) return SI_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_gather_slots(idx, rows, width, lens, row_start, page_table,
                                     page_table ? pages_per_row : 0, page_table ? page_size : 1,
                                     out_slots, stream);
  return e == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}

}  // extern "C"
