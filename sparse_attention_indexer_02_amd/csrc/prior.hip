// Decode path with a threshold from recently selected keys (DoSA reading
// notes, section 1 note on the paper's decoding path: full FP8 scoring is
// kept, and a threshold built mostly from recently selected keys cuts the
// score writeback and the selection work).
//
// Reading: for row r, tau_r is the K-th largest current score among the
// distinct visible keys of the caller's prior list (the keys it selected
// recently), or -inf when fewer than K of them are distinct and visible.
// Those keys are K distinct keys of the row, so the row's K-th largest score
// T_r >= tau_r, and every key of the row's top-K (score > T_r, or == T_r)
// has score >= tau_r.  So:
//   prior_tau     scores the prior keys with the decode micro-kernel (the
//                 same bits the full scoring gives them) -> tau_r;
//   full scoring  every visible key, as idx_score_topk; a 32-key tile writes
//                 a survivor mask (s >= tau_r) and stores survivors' scores;
//   prior_compact survivors in increasing key order with their scores;
//   top-K         over the survivors (position order = key order, so ties
//                 fall to the lower key as in the unfiltered selection).
// The result is idx_score_topk's, bit for bit, whatever the prior; a poor
// prior only costs time.
#include "score_rows.hpp"

namespace si {

constexpr int kPriorMax = 2048;  // prior ids per row
constexpr int kSmallCands = 8192;  // survivors one top-K workgroup takes

template <int MT, int KS, bool FP8>
__global__ __launch_bounds__(256) void prior_tau(
    const uint16_t* __restrict__ q, const void* __restrict__ kv, const float* __restrict__ kscale,
    const float* __restrict__ w, int64_t w_stride, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ vis_len, int64_t n_k, int64_t max_vis, int H,
    const int32_t* __restrict__ prior, int pw, int K, float* __restrict__ tau) {
  constexpr int D = 16 * KS;
  constexpr int ES = FP8 ? 1 : 2;
  constexpr int NL = FP8 ? KS / 2 : KS;
  __shared__ uint64_t srt[kPriorMax];
  __shared__ int ids[kPriorMax];
  __shared__ float sc[kPriorMax];
  __shared__ int hist[2048];
  __shared__ int red[256 / 64 + 8];
  __shared__ int n_dist;
  const int r = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int64_t off;
  const int64_t v = visible_len(vis_len, row_off, r, n_k, max_vis, &off);
  // visible prior ids as id + 1 (0 = none), sorted descending
  const int P = next_pow2(pw);
  for (int i = t; i < P; i += 256) {
    const int64_t id = i < pw ? (int64_t)prior[(int64_t)r * pw + i] : -1;
    srt[i] = (id >= 0 && id < v) ? (uint64_t)(id + 1) : 0ull;
  }
  if (t == 0) n_dist = 0;
  __syncthreads();
  bitonic_sort_desc<256>(srt, P);
  // the distinct ones: the first of each run of equal ids
  for (int i = t; i < P; i += 256)
    if (srt[i] != 0ull && (i == 0 || srt[i] != srt[i - 1])) ids[atomicAdd(&n_dist, 1)] = (int)(srt[i] - 1);
  __syncthreads();
  const int m = n_dist;
  if (m < K) {  // no valid lower bound from this prior: keep every key
    if (t == 0) tau[r] = -__builtin_inff();
    return;
  }
  bf16x8 a[1][MT][KS];
  float wv[MT][16];
  load_rows_frags<MT, KS>(q, w, w_stride, r, H, a, wv);
  for (int tile = wave; tile * 32 < m; tile += 4) {
    const int j = tile * 32 + (lane & 31);
    const int id = ids[j < m ? j : 0];
    const u32x4* kp = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kv) +
                                                     (off + id) * D * ES + (lane >> 5) * (D / 2) * ES);
    u32x4 raw[NL];
#pragma unroll
    for (int c = 0; c < NL; ++c) raw[c] = kp[c];
    const float scl = FP8 ? kscale[off + id] : 1.0f;
    const float s = rows_tile_score<MT, KS, FP8>(a, wv, raw, scl);
    if (lane < 32 && j < m) sc[j] = s;
  }
  __syncthreads();
  int64_t n_gt;
  const uint32_t kk =
      radix_select_kth<256>([&](int64_t i) { return order_key(sc[i]); }, m, K, hist, red, &n_gt);
  if (t == 0) tau[r] = key_to_float(kk);
}

// Survivors of row r in increasing key order, with their scores; rows with
// more than kSmallCands survivors are listed for the chunked selection.
__global__ __launch_bounds__(256) void prior_compact(
    const uint32_t* __restrict__ bitmap, int64_t words, const int32_t* __restrict__ vis_len,
    const int64_t* __restrict__ row_off, int64_t n_k, int64_t max_vis,
    const float* __restrict__ sparse, int64_t sstride, int32_t* __restrict__ cand_ids,
    float* __restrict__ cand_sc, int64_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ ovf, int32_t* __restrict__ ovf_n) {
  __shared__ int red[256 / 64 + 4];
  const int r = blockIdx.x, t = threadIdx.x;
  int64_t off;
  const int64_t v = visible_len(vis_len, row_off, r, n_k, max_vis, &off);
  const int64_t nw = (v + 31) / 32;
  const int64_t per = (nw + 255) / 256;
  const int64_t w0 = t * per, w1 = w0 + per < nw ? w0 + per : nw;
  const uint32_t* bm = bitmap + (int64_t)r * words;
  int c = 0;
  for (int64_t wi = w0; wi < w1; ++wi) c += __builtin_popcount(bm[wi]);
  int tot;
  int64_t pos = block_excl_scan<256>(c, red, &tot);
  for (int64_t wi = w0; wi < w1; ++wi)
    for (uint32_t mb = bm[wi]; mb != 0u; mb &= mb - 1u) {
      const int64_t id = 32 * wi + __builtin_ctz(mb);
      cand_ids[(int64_t)r * cap + pos] = (int32_t)id;
      cand_sc[(int64_t)r * cap + pos] = sparse[(int64_t)r * sstride + id];
      ++pos;
    }
  if (t == 0) {
    counts[r] = tot;
    if (tot > kSmallCands) ovf[atomicAdd(ovf_n, 1)] = r;
  }
}

__global__ void prior_zero(int32_t* p) { *p = 0; }

// Workspace regions (256-byte aligned): tau, bitmap, sparse scores, the
// candidates, counts, the overflow list, the chunked top-K's levels.
struct PriorLayout {
  size_t tau, bitmap, sparse, cand_ids, cand_sc, counts, ovf, topk_ws, total;
  int64_t words, cap;
  size_t topk_ws_bytes;
};
static PriorLayout prior_layout(int64_t n_q, int64_t max_vis, int K) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  PriorLayout L{};
  L.words = (max_vis + 31) / 32;
  L.cap = max_vis;
  size_t o = 0;
  L.tau = o; o += al((size_t)n_q * 4);
  L.bitmap = o; o += al((size_t)n_q * L.words * 4);
  L.sparse = o; o += al((size_t)n_q * max_vis * 4);
  L.cand_ids = o; o += al((size_t)n_q * L.cap * 4);
  L.cand_sc = o; o += al((size_t)n_q * L.cap * 4);
  L.counts = o; o += al((size_t)n_q * 4);
  L.ovf = o; o += al((size_t)(n_q + 1) * 4);
  L.topk_ws = o;
  L.topk_ws_bytes = topk_workspace_bytes(n_q, L.cap, K);
  o += al(L.topk_ws_bytes);
  L.total = o;
  return L;
}

size_t prior_workspace_bytes(int64_t n_q, int64_t max_vis, int K) {
  if (n_q <= 0 || max_vis <= 0) return 0;
  return prior_layout(n_q, max_vis, K).total;
}

template <int MT, int KS>
static hipError_t run_prior(const ScoreArgs& sa, const int32_t* prior, int pw, int K,
                            int32_t* out_idx, float* out_score, float* out_tau,
                            int32_t* out_count, unsigned char* ws, hipStream_t st) {
  const PriorLayout L = prior_layout(sa.n_q, sa.max_vis, K);
  float* tau = reinterpret_cast<float*>(ws + L.tau);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws + L.bitmap);
  float* sparse = reinterpret_cast<float*>(ws + L.sparse);
  int32_t* cand_ids = reinterpret_cast<int32_t*>(ws + L.cand_ids);
  float* cand_sc = reinterpret_cast<float*>(ws + L.cand_sc);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* ovf = reinterpret_cast<int32_t*>(ws + L.ovf);
  int32_t* ovf_n = ovf + sa.n_q;
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(sa.q);
  if (sa.k_dtype == SI_FP8_E4M3FN)
    hipLaunchKernelGGL((prior_tau<MT, KS, true>), dim3(sa.n_q), dim3(256), 0, st, q16, sa.k,
                       sa.k_scale, sa.w, sa.w_row_stride, sa.k_row_offset, sa.vis_len, sa.n_k,
                       sa.max_vis, sa.H, prior, pw, K, tau);
  else
    hipLaunchKernelGGL((prior_tau<MT, KS, false>), dim3(sa.n_q), dim3(256), 0, st, q16, sa.k,
                       sa.k_scale, sa.w, sa.w_row_stride, sa.k_row_offset, sa.vis_len, sa.n_k,
                       sa.max_vis, sa.H, prior, pw, K, tau);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScoreArgs fa = sa;
  fa.scores = sparse;
  fa.score_stride = sa.max_vis;
  fa.filter_tau = tau;
  fa.filter_bitmap = bitmap;
  fa.filter_words = L.words;
  e = launch_score(fa, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prior_zero, dim3(1), dim3(1), 0, st, ovf_n);
  hipLaunchKernelGGL(prior_compact, dim3(sa.n_q), dim3(256), 0, st, bitmap, L.words, sa.vis_len,
                     sa.k_row_offset, sa.n_k, sa.max_vis, sparse, sa.max_vis, cand_ids, cand_sc,
                     L.cap, counts, ovf, ovf_n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // every row through one workgroup over its first kSmallCands survivors;
  // rows with more are then redone by the chunked selection over all of them
  TopkArgs ta;
  ta.scores = cand_sc; ta.stride = L.cap; ta.vis_len = counts; ta.k_row_offset = nullptr;
  ta.n_k = L.cap; ta.n_rows = sa.n_q; ta.K = K; ta.out_idx = out_idx; ta.out_score = out_score;
  ta.id_map = cand_ids; ta.id_map_stride = L.cap;
  const bool split = K <= 2048 && L.cap > kSmallCands;
  ta.max_vis = split ? kSmallCands : L.cap;
  ta.workspace = ws + L.topk_ws;
  ta.workspace_bytes = L.topk_ws_bytes;
  e = launch_topk(ta, st);
  if (e != hipSuccess) return e;
  if (split) {
    TopkArgs tb = ta;
    tb.max_vis = L.cap;
    tb.row_list = ovf;
    tb.row_count = ovf_n;
    e = launch_topk(tb, st);
    if (e != hipSuccess) return e;
  }
  if (out_tau) {
    e = hipMemcpyAsync(out_tau, tau, (size_t)sa.n_q * 4, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
  }
  if (out_count) {
    e = hipMemcpyAsync(out_count, counts, (size_t)sa.n_q * 4, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_prior_topk(const ScoreArgs& sa, const int32_t* prior, int pw, int K,
                             int32_t* out_idx, float* out_score, float* out_tau,
                             int32_t* out_count, void* ws, hipStream_t st) {
  if (sa.n_q == 0) return hipSuccess;
  unsigned char* w = static_cast<unsigned char*>(ws);
  const int MT = sa.H <= 32 ? 1 : 2;
  if (sa.D == 128)
    return MT == 1 ? run_prior<1, 8>(sa, prior, pw, K, out_idx, out_score, out_tau, out_count, w, st)
                   : run_prior<2, 8>(sa, prior, pw, K, out_idx, out_score, out_tau, out_count, w, st);
  return MT == 1 ? run_prior<1, 4>(sa, prior, pw, K, out_idx, out_score, out_tau, out_count, w, st)
                 : run_prior<2, 4>(sa, prior, pw, K, out_idx, out_score, out_tau, out_count, w, st);
}

}  // namespace si
