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
//   prior_score   scores the distinct prior keys with the decode micro-kernel
//   + prior_kth   (the same bits the full scoring gives them) -> tau_r
//                 (prior_tau, one workgroup per row, for rows too long for
//                 an LDS bitmap of their keys);
//   full scoring  every visible key, as idx_score_topk; a 32-key tile writes
//                 a survivor mask (s >= tau_r) and stores survivors' scores,
//                 and each key chunk its survivor count;
//   prior_compact survivors in increasing key order with their scores, one
//                 workgroup per key chunk;
//   top-K         over the survivors (position order = key order, so ties
//                 fall to the lower key as in the unfiltered selection).
// The result is idx_score_topk's, bit for bit, whatever the prior; a poor
// prior only costs time.
#include "score_rows.hpp"

namespace si {

constexpr int kPriorMax = 2048;  // prior ids per row
constexpr int kSmallCands = kBlockTopkMaxN;  // survivors one top-K workgroup takes

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

// The same tau with the row's work spread over kPriorSplit workgroups, for
// rows of at most kPriorBitmapKeys keys: every workgroup marks the visible
// prior ids in an LDS bitmap of the row (repeats collapse; dynamic LDS of
// (max_vis + 31) / 32 words), and scores the
// distinct ids of its share of the bitmap words, in id order, into slots
// (rank among the distinct ids) of prior_sc [n_q, kPriorMax]; workgroup 0
// records their number m.  prior_kth then takes the K-th largest.
constexpr int kPriorSplit = 4;
constexpr int64_t kPriorBitmapKeys = 1 << 18;  // at most 32 KB of LDS bits

template <int MT, int KS, bool FP8>
__global__ __launch_bounds__(256) void prior_score(
    const uint16_t* __restrict__ q, const void* __restrict__ kv, const float* __restrict__ kscale,
    const float* __restrict__ w, int64_t w_stride, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ vis_len, int64_t n_k, int64_t max_vis, int H,
    const int32_t* __restrict__ prior, int pw, int K, float* __restrict__ prior_sc,
    int32_t* __restrict__ prior_m) {
  constexpr int D = 16 * KS;
  constexpr int ES = FP8 ? 1 : 2;
  constexpr int NL = FP8 ? KS / 2 : KS;
  extern __shared__ uint32_t bits[];
  __shared__ int ids[kPriorMax];
  __shared__ int red[256 / 64 + 4];
  const int r = blockIdx.x, part = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int64_t off;
  const int64_t v = visible_len(vis_len, row_off, r, n_k, max_vis, &off);  // <= kPriorBitmapKeys
  const int nw = (int)((v + 31) / 32);
  // global reads first (the prior ids, then the row's query fragments), so
  // their latency overlaps the bitmap work
  int pid[kPriorMax / 256];
#pragma unroll
  for (int k = 0; k < kPriorMax / 256; ++k) {
    const int i = t + 256 * k;
    pid[k] = i < pw ? prior[(int64_t)r * pw + i] : -1;
  }
  bf16x8 a[1][MT][KS];
  float wv[MT][16];
  load_rows_frags<MT, KS>(q, w, w_stride, r, H, a, wv);
  for (int i = t; i < nw; i += 256) bits[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPriorMax / 256; ++k)
    if (pid[k] >= 0 && pid[k] < v) atomicOr(&bits[pid[k] >> 5], 1u << (pid[k] & 31));
  __syncthreads();
  // this part's words [w0, w1); distinct ids before them and in the row
  const int per = (nw + kPriorSplit - 1) / kPriorSplit;
  const int w0 = part * per < nw ? part * per : nw;
  const int w1 = w0 + per < nw ? w0 + per : nw;
  int before = 0, all = 0;
  for (int i = t; i < nw; i += 256) {
    const int c = __builtin_popcount(bits[i]);
    before += i < w0 ? c : 0;
    all += c;
  }
  int m_before, m;
  (void)block_excl_scan<256>(before, red, &m_before);
  (void)block_excl_scan<256>(all, red, &m);
  if (part == 0 && t == 0) prior_m[r] = m;
  if (m < K) return;  // tau is -inf: nothing to score
  // ids of this part in increasing order: thread t takes a run of its words
  const int wpt = (w1 - w0 + 255) / 256;
  const int a0 = w0 + t * wpt < w1 ? w0 + t * wpt : w1;
  const int a1 = a0 + wpt < w1 ? a0 + wpt : w1;
  int mine = 0;
  for (int i = a0; i < a1; ++i) mine += __builtin_popcount(bits[i]);
  int n_part;
  int pos = block_excl_scan<256>(mine, red, &n_part);
  for (int i = a0; i < a1; ++i)
    for (uint32_t mb = bits[i]; mb != 0u; mb &= mb - 1u) ids[pos++] = 32 * i + __builtin_ctz(mb);
  __syncthreads();
  if (n_part == 0) return;
  // 32 ids per tile, tiles wave + 4 i; the next tile's keys load during
  // each tile's MFMAs
  auto kload = [&](int tile, u32x4 (&raw)[NL], float& scl) {
    const int j = tile * 32 + (lane & 31);
    const int id = ids[j < n_part ? j : 0];
    const u32x4* kp = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kv) +
                                                     (off + id) * D * ES + (lane >> 5) * (D / 2) * ES);
#pragma unroll
    for (int c = 0; c < NL; ++c) raw[c] = kp[c];
    scl = FP8 ? kscale[off + id] : 1.0f;
  };
  u32x4 ra[NL], rb[NL];
  float sa = 1.0f, sb = 1.0f;
  if (wave * 32 < n_part) kload(wave, ra, sa);
  for (int tile = wave; tile * 32 < n_part; tile += 4) {
    if ((tile + 4) * 32 < n_part) kload(tile + 4, rb, sb);
    const float s = rows_tile_score<MT, KS, FP8>(a, wv, ra, sa);
    const int j = tile * 32 + (lane & 31);
    if (lane < 32 && j < n_part) prior_sc[(int64_t)r * kPriorMax + m_before + j] = s;
#pragma unroll
    for (int c = 0; c < NL; ++c) ra[c] = rb[c];
    sa = sb;
  }
}

// tau_r: the K-th largest of the row's m distinct prior scores (their
// minimum when m == K, as for a prior of the last step's K ids), -inf when
// m < K.  Workgroup 0 also clears the overflow row count for prior_compact.
__global__ __launch_bounds__(256) void prior_kth(const float* __restrict__ prior_sc,
                                                 const int32_t* __restrict__ prior_m, int K,
                                                 float* __restrict__ tau, int32_t* __restrict__ ovf_n) {
  __shared__ uint32_t keys[kPriorMax];
  __shared__ int hist[2048];
  __shared__ int red[256 / 64 + 8];
  const int r = blockIdx.x;
  if (r == 0 && threadIdx.x == 0) *ovf_n = 0;
  const int m = prior_m[r];
  if (m < K) {
    if (threadIdx.x == 0) tau[r] = -__builtin_inff();
    return;
  }
  const float* ps = prior_sc + (int64_t)r * kPriorMax;
  if (m == K) {
    uint32_t lo = 0xFFFFFFFFu;
    for (int i = threadIdx.x; i < m; i += 256) {
      const uint32_t u = order_key(ps[i]);
      lo = u < lo ? u : lo;
    }
    lo = __ockl_wfred_min_u32(lo);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = (int)lo;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t b = (uint32_t)red[0];
      for (int i = 1; i < 4; ++i) b = (uint32_t)red[i] < b ? (uint32_t)red[i] : b;
      tau[r] = key_to_float(b);
    }
    return;
  }
  for (int i = threadIdx.x; i < m; i += 256) keys[i] = order_key(ps[i]);
  __syncthreads();
  int64_t n_gt;
  const uint32_t kk =
      radix_select_kth<256>([&](int64_t i) { return keys[i]; }, m, K, hist, red, &n_gt);
  if (threadIdx.x == 0) tau[r] = key_to_float(kk);
}

// Survivors of row r in increasing key order, with their scores: workgroup
// (r, c) takes key chunk c, whose survivors start after those of the chunks
// before it (chunk_cnt [n_q, chunks, 4]: the counts of a chunk's waves);
// thread t takes keys t + 256 i of the chunk (coalesced reads of the
// scores).  Workgroup (r, 0) records the row's count and lists rows
// with more than kSmallCands survivors for the chunked selection.
__global__ __launch_bounds__(256) void prior_compact(
    const uint32_t* __restrict__ bitmap, int64_t words, const int32_t* __restrict__ chunk_cnt,
    int64_t chunks, const int32_t* __restrict__ vis_len, const int64_t* __restrict__ row_off,
    int64_t n_k, int64_t max_vis, const float* __restrict__ sparse, int64_t sstride,
    int32_t* __restrict__ cand_ids, float* __restrict__ cand_sc, int64_t cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ ovf, int32_t* __restrict__ ovf_n) {
  constexpr int CW = kRowsChunk / 32;  // bitmap words per chunk
  __shared__ uint32_t wb[CW];
  __shared__ int wpre[CW];
  __shared__ int red[256 / 64 + 4];
  const int r = rows_grid_row(), t = threadIdx.x;
  const int64_t c = blockIdx.y;
  // the chunk's bitmap words and the row's chunk counts are read before the
  // row's length arrives (entries past it are masked below)
  const int64_t wi = c * CW + t;
  const uint32_t mb_raw = (t < CW && wi < words) ? bitmap[(int64_t)r * words + wi] : 0u;
  // chunk i's count: the sum of its four waves' counts
  const int4* cc = reinterpret_cast<const int4*>(chunk_cnt) + (int64_t)r * chunks;
  auto chunk_total = [&](int64_t i) {
    const int4 x = cc[i];
    return x.x + x.y + x.z + x.w;
  };
  const int cc_raw = t < chunks ? chunk_total(t) : 0;
  int64_t off;
  const int64_t v = visible_len(vis_len, row_off, r, n_k, max_vis, &off);
  const int64_t nch = (v + kRowsChunk - 1) / kRowsChunk;
  if (c >= nch && c > 0) return;  // chunk 0 still records an empty row's count
  const int64_t c0 = c * kRowsChunk;
  const uint32_t mb = wi < (v + 31) / 32 ? mb_raw : 0u;
  int pre = 0, all = 0;
  for (int64_t i = t; i < nch; i += 256) {
    const int x = i == t ? cc_raw : chunk_total(i);
    pre += i < c ? x : 0;
    all += x;
  }
  int base;
  (void)block_excl_scan<256>(pre, red, &base);
  if (c == 0) {
    int tot;
    (void)block_excl_scan<256>(all, red, &tot);
    if (t == 0) {
      counts[r] = tot;
      if (tot > kSmallCands) ovf[atomicAdd(ovf_n, 1)] = r;
    }
  }
  int n_chunk;
  const int wp = block_excl_scan<256>(__builtin_popcount(mb), red, &n_chunk);
  if (t < CW) {
    wb[t] = mb;
    wpre[t] = wp;
  }
  __syncthreads();
  if (n_chunk == 0) return;
  int32_t* oi = cand_ids + (int64_t)r * cap + base;
  float* os = cand_sc + (int64_t)r * cap + base;
  const float* sp = sparse + (int64_t)r * sstride + c0;
  // keys t + 256 i: the survivors' scores are all requested before any is
  // written
  constexpr int NI = kRowsChunk / 256;
  uint32_t word[NI];
  float val[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = t + 256 * i;
    word[i] = wb[j >> 5];
    val[i] = ((word[i] >> (j & 31)) & 1u) ? sp[j] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = t + 256 * i;
    if ((word[i] >> (j & 31)) & 1u) {
      const int pos = wpre[j >> 5] + __builtin_popcount(word[i] & ((1u << (j & 31)) - 1u));
      oi[pos] = (int32_t)(c0 + j);
      os[pos] = val[i];
    }
  }
}

__global__ void prior_zero(int32_t* p) { *p = 0; }

// Workspace regions (256-byte aligned): tau, bitmap, per-chunk survivor
// counts, the prior scores and their counts, sparse scores, the candidates,
// counts, the overflow list, the chunked top-K's levels.
struct PriorLayout {
  size_t tau, bitmap, chunk_cnt, prior_sc, prior_m, sparse, cand_ids, cand_sc, counts, ovf,
      topk_ws, total;
  int64_t words, chunks, cap;
  size_t topk_ws_bytes;
};
static PriorLayout prior_layout(int64_t n_q, int64_t max_vis, int K) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  PriorLayout L{};
  L.words = (max_vis + 31) / 32;
  L.chunks = rows_key_chunks(max_vis);
  L.cap = max_vis;
  size_t o = 0;
  L.tau = o; o += al((size_t)n_q * 4);
  L.bitmap = o; o += al((size_t)n_q * L.words * 4);
  L.chunk_cnt = o; o += al((size_t)n_q * L.chunks * 16);
  L.prior_sc = o; o += al((size_t)n_q * kPriorMax * 4);
  L.prior_m = o; o += al((size_t)n_q * 4);
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
  int32_t* chunk_cnt = reinterpret_cast<int32_t*>(ws + L.chunk_cnt);
  float* prior_sc = reinterpret_cast<float*>(ws + L.prior_sc);
  int32_t* prior_m = reinterpret_cast<int32_t*>(ws + L.prior_m);
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(sa.q);
  const bool fp8 = sa.k_dtype == SI_FP8_E4M3FN;
  if (sa.max_vis <= kPriorBitmapKeys) {
    const dim3 g2((unsigned)sa.n_q, kPriorSplit);
    const size_t lds = (size_t)L.words * 4;
    if (fp8)
      hipLaunchKernelGGL((prior_score<MT, KS, true>), g2, dim3(256), lds, st, q16, sa.k, sa.k_scale,
                         sa.w, sa.w_row_stride, sa.k_row_offset, sa.vis_len, sa.n_k, sa.max_vis,
                         sa.H, prior, pw, K, prior_sc, prior_m);
    else
      hipLaunchKernelGGL((prior_score<MT, KS, false>), g2, dim3(256), lds, st, q16, sa.k, sa.k_scale,
                         sa.w, sa.w_row_stride, sa.k_row_offset, sa.vis_len, sa.n_k, sa.max_vis,
                         sa.H, prior, pw, K, prior_sc, prior_m);
    hipLaunchKernelGGL(prior_kth, dim3(sa.n_q), dim3(256), 0, st, prior_sc, prior_m, K, tau, ovf_n);
  } else if (fp8) {
    hipLaunchKernelGGL((prior_tau<MT, KS, true>), dim3(sa.n_q), dim3(256), 0, st, q16, sa.k,
                       sa.k_scale, sa.w, sa.w_row_stride, sa.k_row_offset, sa.vis_len, sa.n_k,
                       sa.max_vis, sa.H, prior, pw, K, tau);
  } else {
    hipLaunchKernelGGL((prior_tau<MT, KS, false>), dim3(sa.n_q), dim3(256), 0, st, q16, sa.k,
                       sa.k_scale, sa.w, sa.w_row_stride, sa.k_row_offset, sa.vis_len, sa.n_k,
                       sa.max_vis, sa.H, prior, pw, K, tau);
  }
  if (sa.max_vis > kPriorBitmapKeys) hipLaunchKernelGGL(prior_zero, dim3(1), dim3(1), 0, st, ovf_n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScoreArgs fa = sa;
  fa.scores = sparse;
  fa.score_stride = sa.max_vis;
  fa.filter_tau = tau;
  fa.filter_bitmap = bitmap;
  fa.filter_words = L.words;
  fa.filter_chunk_cnt = chunk_cnt;
  e = launch_score(fa, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prior_compact, dim3((unsigned)sa.n_q, (unsigned)L.chunks), dim3(256), 0, st,
                     bitmap, L.words, chunk_cnt, L.chunks, sa.vis_len, sa.k_row_offset, sa.n_k,
                     sa.max_vis, sparse, sa.max_vis, cand_ids, cand_sc, L.cap, counts, ovf, ovf_n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // every row through one workgroup over its first kSmallCands survivors;
  // rows with more (listed by prior_compact) are then redone over all of
  // them by the chunked selection (8192-survivor chunks, then merge levels),
  // whose launches end at once when no row is listed
  TopkArgs ta;
  ta.scores = cand_sc; ta.stride = L.cap; ta.vis_len = counts; ta.k_row_offset = nullptr;
  ta.n_k = L.cap; ta.n_rows = sa.n_q; ta.K = K; ta.out_idx = out_idx; ta.out_score = out_score;
  ta.id_map = cand_ids; ta.id_map_stride = L.cap;
  ta.workspace = ws + L.topk_ws;
  ta.workspace_bytes = L.topk_ws_bytes;
  if (K <= kBlockTopkMaxK && L.cap > kSmallCands) {
    ta.max_vis = kSmallCands;
    e = launch_topk(ta, st);
    if (e != hipSuccess) return e;
    TopkArgs tb = ta;
    tb.max_vis = L.cap;
    tb.row_list = ovf;
    tb.row_count = ovf_n;
    e = launch_topk(tb, st);
  } else {
    ta.max_vis = L.cap;  // one workgroup per row takes it whole (larger K: the radix select)
    e = launch_topk(ta, st);
  }
  if (e != hipSuccess) return e;
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
