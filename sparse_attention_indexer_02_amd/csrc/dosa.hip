// DoSA certified prune (DoSA reading notes, sections 2-4), prefill layout.
//
// Pipeline, all on the caller's stream, every grid sized from host-known
// bounds (no device-to-host reads):
//   init        common visible prefix c, flags, zeroed counters
//   cold prior  representative rows t_i = round(i (n_q-1)/(R-1)) scored over
//               [0, c) and top-rep_topk'd; key occurrence counts; seeds =
//               n_seeds keys of [0, c) by (count desc, key asc), kept in
//               ascending key order (section 4).  A caller prior replaces it.
//   seed pass   every row x every seed with the shared score micro-kernel;
//               seed top-K by (score desc, key asc); tau = its K-th score
//               (section 2.1).  Before it, per-head activation counts and
//               ReLU sums over a sample of 128 seeds evenly spaced in seed
//               order (section 4: activation patterns from 128 positions of
//               the seed region).
//   plan        per row: kept heads = the kept_heads largest
//               |w_h| * mean_sample max(x_h, 0); each omitted positive head
//               anchors on the kept head of smallest residual under the
//               clamped projection beta = max(0, q_h.q_j/|q_j|^2) (section
//               3.1); folded weights w'_j = w_j + sum beta_h w_h; residual
//               R = sum w_h |d_h|; omitted negative heads active on at least
//               neg_active_frac of the sample aggregate into a_A = sum |w_h| q_h
//               (section 3.2), carried in bf16 as a_hat.  All in fp64.
//   bound       MFMA over the 32-row plan tile (kept heads, a_hat, zeros):
//               U = sum w'_j max(x_j,0) - max(a_hat.k, 0) + C_r |k|; a key
//               survives iff U >= tau (section 2.2).  C_r = R + |a_A - a_hat|
//               + 2^-10 (sum_h |w_h||q_h| + sum_J |w'_j||q_j| + |a_hat| + R +
//               |a_A - a_hat|): ReLU is 1-Lipschitz, so the a_hat term costs
//               |a_A - a_hat||k|, and 2^-10 |.||k| dominates every fp32
//               rounding of the computed score and of U (fp32 MFMA sums of
//               128 exact products err by at most ~2^-16 |q||k|).  So U is
//               at least the score this device computes.
//   compact     ballot bitmap -> ascending survivor ids; more than
//               survivor_capacity sends the row to the exact path.  The
//               bound scan keeps a running survivor count per row and
//               skips the rest of a row once it passes the capacity (the
//               exact path will score every key of it anyway); the count
//               then decides the row's fallback.
//               With shared streams (section 4's compaction variant): rows
//               go in groups of 4; a key that survives for at least 2 of
//               the group's rows and lies in the group's common visible
//               prefix goes to the group's shared stream, every other
//               survivor to its row's solo stream (rows over the capacity
//               take the exact path and no part in the split).
//   rescore     survivors with the shared micro-kernel; keep s >= tau.  A
//               shared stream's key tile is fetched once into LDS and scored
//               for all 4 rows (one wave per row); a row keeps a shared key
//               iff its own s >= tau (a key whose bound failed for the row
//               has s <= U < tau, so this adds nothing wrong).
//   merge       seed top-K (sorted) merged with the sorted kept survivors;
//               first K by (score desc, key asc).
//   fallback    listed rows (overflow, or every row when c < n_seeds or a
//               caller prior is invalid) take the unpruned score + top-K.
// The result equals idx_score_topk's bit for bit: scores come from one
// micro-kernel, and every key of the unpruned top-K is a seed in the seed
// top-K or a survivor with s >= tau (its U >= s >= K-th overall >= tau).
#include <math.h>

#include "score_micro.hpp"

namespace si {

struct DosaCtx {
  int32_t c;                // common visible prefix
  int32_t global_fallback;  // every row takes the exact path
  int32_t n_fallback;       // length of the fallback row list
  int32_t pad[61];
};

struct DosaLayout {
  size_t ctx, rep_q, rep_w, rep_vis, rep_scores, rep_ids, counts, seeds, seed_mask, seed_keys, sample_keys,
      seed_scores, stat_cnt, stat_sum, top_idx, top_score, plan_a, plan_w, plan_c, knorm, bitmap,
      surv_ids, surv_cnt, bound_cnt, row_fb, kept_score, kept_id, kept_cnt, fb_list, fb_scores, shared_ids,
      shared_cnt, solo_cnt, shared_n, topk_ws, topk_ws_bytes, total;
};

static size_t au(size_t x) { return (x + 255) / 256 * 256; }

// Activation statistics sample: 128 seeds (all of them when there are
// fewer), evenly spaced in seed order (DoSA reading notes, section 4: the
// planner counts activation patterns over 128 positions of the seed region).
constexpr int kStatSample = 128;
__host__ __device__ inline int stat_sample_size(int n_seeds) {
  return n_seeds < kStatSample ? n_seeds : kStatSample;
}
// Seed index of sample i of m: round(i (n_seeds - 1) / (m - 1)), halves up.
__host__ __device__ inline int stat_sample_index(int i, int m, int n_seeds) {
  return m > 1 ? (int)((2LL * i * (n_seeds - 1) + (m - 1)) / (2LL * (m - 1))) : 0;
}

static DosaLayout dosa_layout(int32_t n_q, int32_t H, int32_t D, int64_t n_k, int32_t topk,
                              const si_dosa_params* p) {
  DosaLayout L;
  size_t o = 0;
  const size_t nq = (size_t)n_q, nk = (size_t)n_k, R = (size_t)p->n_rep_queries;
  const size_t ns = (size_t)p->n_seeds, cap = (size_t)p->survivor_capacity;
  const size_t words = (nk + 31) / 32;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += au(bytes);
    return at;
  };
  L.ctx = take(sizeof(DosaCtx));
  L.rep_q = take(R * H * D * 2);
  L.rep_w = take(R * H * 4);
  L.rep_vis = take(R * 4);
  L.rep_scores = take(R * nk * 4);
  L.rep_ids = take(R * (size_t)p->rep_topk * 4);
  L.counts = take(nk * 4);
  L.seeds = take(ns * 4);
  L.seed_mask = take(words * 4);
  L.seed_keys = take(ns * D * 2);
  L.sample_keys = take((size_t)kStatSample * D * 2);
  L.seed_scores = take(nq * ns * 4);
  L.stat_cnt = take(nq * H * 4);
  L.stat_sum = take(nq * H * 4);
  L.top_idx = take(nq * topk * 4);
  L.top_score = take(nq * topk * 4);
  L.plan_a = take(nq * 32 * D * 2);
  L.plan_w = take(nq * 32 * 4);
  L.plan_c = take(nq * 4);
  L.knorm = take(nk * 4);
  L.bitmap = take(nq * words * 4);
  L.surv_ids = take(nq * cap * 4);
  L.surv_cnt = take(nq * 4);
  L.bound_cnt = take(nq * 4);
  L.row_fb = take(nq * 4);
  L.kept_score = take(nq * cap * 4);
  L.kept_id = take(nq * cap * 4);
  L.kept_cnt = take(nq * 4);
  L.fb_list = take(nq * 4);
  L.fb_scores = take(nq * nk * 4);
  // 4-query groups: shared streams [groups, 2 cap], their lengths, each
  // row's solo stream length and its survivors taken through the shared
  // stream
  const size_t ng = (nq + 3) / 4;
  L.shared_ids = take(ng * 2 * cap * 4);
  L.shared_cnt = take(ng * 4);
  L.solo_cnt = take(nq * 4);
  L.shared_n = take(nq * 4);
  // candidate lists of the chunked top-K, shared by its three uses (the
  // representative rows, the seed rows and the exact-path rows run one
  // after the other)
  {
    size_t w = topk_workspace_bytes(R, nk, p->rep_topk);
    const size_t w2 = topk_workspace_bytes(nq, ns, topk);
    const size_t w3 = topk_workspace_bytes(nq, nk, topk);
    w = w2 > w ? w2 : w;
    w = w3 > w ? w3 : w;
    L.topk_ws_bytes = w;
    L.topk_ws = take(w);
  }
  L.total = o;
  return L;
}

constexpr int kMaxRep = 64;
constexpr int kMaxCapacity = 8192;

// ---------------------------------------------------------------------------
__global__ void fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ __launch_bounds__(1024) void dosa_init(DosaCtx* ctx, const int32_t* vis_len, int n_q,
                                                  int64_t n_k, int n_seeds, int32_t* rep_vis,
                                                  int R) {
  __shared__ int red[32];
  int m = INT32_MAX;
  for (int r = threadIdx.x; r < n_q; r += 1024) {
    int64_t off;
    int v = (int)visible_len(vis_len, nullptr, r, n_k, n_k, &off);
    m = v < m ? v : m;
  }
  for (int o = 32; o > 0; o >>= 1) {
    int y = __shfl_xor(m, o, 64);
    m = y < m ? y : m;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = INT32_MAX;
    for (int i = 0; i < 1024 / 64; ++i) c = red[i] < c ? red[i] : c;
    if (n_q == 0) c = 0;
    ctx->c = c;
    ctx->global_fallback = (c < n_seeds) ? 1 : 0;
    ctx->n_fallback = 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R; i += 1024) rep_vis[i] = ctx->c;
}

// Representative rows t_i = round(i (n_q - 1) / (R - 1)), gathered densely.
__global__ __launch_bounds__(256) void dosa_gather_rep(const uint16_t* q, const float* w,
                                                       int64_t w_stride, int n_q, int H, int D,
                                                       int R, uint16_t* rep_q, float* rep_w) {
  const int i = blockIdx.x;
  int t = 0;
  if (R > 1 && n_q > 1)
    t = (int)((2LL * i * (n_q - 1) + (R - 1)) / (2LL * (R - 1)));
  for (int e = threadIdx.x; e < H * D; e += 256) rep_q[(int64_t)i * H * D + e] =
      q[(int64_t)t * H * D + e];
  for (int h = threadIdx.x; h < H; h += 256) rep_w[(int64_t)i * H + h] = w[(int64_t)t * w_stride + h];
}

__global__ void dosa_count(const int32_t* rep_ids, int64_t n, int32_t* counts, int64_t n_k) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int id = rep_ids[i];
    if (id >= 0 && id < n_k) atomicAdd(&counts[id], 1);
  }
}

// Seeds: the caller's (validated) or the first n_seeds keys of [0, c) by
// (count desc, key asc), written ascending; the seed bitmap is set.
constexpr int kSelLdsKeys = 40960;  // common prefixes up to this many keys stage their counts in LDS
__global__ __launch_bounds__(1024) void dosa_select_seeds(DosaCtx* ctx, const int32_t* counts,
                                                          int R, int n_seeds,
                                                          const int32_t* caller_seeds,
                                                          int32_t* seeds, uint32_t* seed_mask) {
  constexpr int T = 1024;
  __shared__ int ge[kMaxRep + 2];
  __shared__ int red[T / 64 + 4];
  __shared__ int bad;
  if (ctx->global_fallback) return;
  const int c = ctx->c;
  if (caller_seeds) {
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n_seeds; i += T) {
      int id = caller_seeds[i];
      bool ok = id >= 0 && id < c && (i == 0 || caller_seeds[i - 1] < id);
      if (!ok) bad = 1;
      seeds[i] = ok ? id : 0;
      if (ok) atomicOr(&seed_mask[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    if (threadIdx.x == 0 && bad) ctx->global_fallback = 1;
    return;
  }
  // per-wave histograms of the counts (atomics contend within a wave only),
  // then ge[v] := #{count >= v}.  The clamped counts (<= kMaxRep) are also
  // kept as bytes in LDS when the prefix fits, so the passes below, where a
  // thread walks its own run of keys, read LDS rather than strided global
  // memory.
  __shared__ int hw[T / 64][kMaxRep + 2];
  __shared__ uint8_t cb[kSelLdsKeys];
  const bool staged = c <= kSelLdsKeys;
  const int wv = threadIdx.x >> 6;
  for (int v = threadIdx.x & 63; v <= R + 1; v += 64) hw[wv][v] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < c; j += T) {
    int cnt = counts[j];
    cnt = cnt > R ? R : cnt;
    atomicAdd(&hw[wv][cnt], 1);
    if (staged) cb[j] = (uint8_t)cnt;
  }
  __syncthreads();
  for (int v = threadIdx.x; v <= R + 1; v += T) {
    int sum = 0;
    for (int w2 = 0; w2 < T / 64; ++w2) sum += hw[w2][v];
    ge[v] = sum;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int v = R - 1; v >= 0; --v) ge[v] += ge[v + 1];
  __syncthreads();
  int vstar = 0;
  for (int v = R; v >= 0; --v)
    if (ge[v] >= n_seeds) {
      vstar = v;
      break;
    }
  const int need_eq = n_seeds - ge[vstar + 1];  // taken among count == vstar, by key
  // thread t owns the keys [t per, (t + 1) per): one scan of its count == vstar
  // keys gives their index-order ranks, one scan of its selected keys their
  // output slots (the seed list is in increasing key order)
  const int per = (c + T - 1) / T;
  const int j0 = (int)threadIdx.x * per, j1 = j0 + per < c ? j0 + per : c;
  auto cnt_of = [&](int j) { return staged ? (int)cb[j] : (counts[j] > R ? R : counts[j]); };
  int n_eq = 0;
  for (int j = j0; j < j1; ++j) n_eq += cnt_of(j) == vstar ? 1 : 0;
  int tot;
  const int eq_base = block_excl_scan<T>(n_eq, red, &tot);
  int n_sel = 0;
  for (int j = j0, er = eq_base; j < j1; ++j) {
    const int v = cnt_of(j);
    n_sel += (v > vstar || (v == vstar && er < need_eq)) ? 1 : 0;
    er += v == vstar ? 1 : 0;
  }
  int pos = block_excl_scan<T>(n_sel, red, &tot);
  for (int j = j0, er = eq_base; j < j1; ++j) {
    const int v = cnt_of(j);
    if (v > vstar || (v == vstar && er < need_eq)) {
      seeds[pos++] = j;
      atomicOr(&seed_mask[j >> 5], 1u << (j & 31));
    }
    er += v == vstar ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void dosa_gather_seed_keys(const DosaCtx* ctx,
                                                             const uint16_t* k,
                                                             const int32_t* seeds, int n_seeds,
                                                             int D, uint16_t* seed_keys) {
  if (ctx->global_fallback) return;
  const int cpk = D / 8;  // 16-byte chunks per key
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < (int64_t)n_seeds * cpk;
       e += (int64_t)gridDim.x * 256) {
    int i = (int)(e / cpk), c = (int)(e % cpk);
    reinterpret_cast<u32x4*>(seed_keys + (int64_t)i * D)[c] =
        reinterpret_cast<const u32x4*>(k + (int64_t)seeds[i] * D)[c];
  }
}

__global__ __launch_bounds__(256) void dosa_gather_sample(const DosaCtx* ctx, const uint16_t* k,
                                                          const int32_t* seeds, int n_seeds,
                                                          int D, uint16_t* sample_keys) {
  if (ctx->global_fallback) return;
  const int m = stat_sample_size(n_seeds);
  const int cpk = D / 8;  // 16-byte chunks per key
  for (int e = threadIdx.x; e < m * cpk; e += 256) {
    const int i = e / cpk, c = e % cpk;
    const int j = seeds[stat_sample_index(i, m, n_seeds)];
    reinterpret_cast<u32x4*>(sample_keys + (int64_t)i * D)[c] =
        reinterpret_cast<const u32x4*>(k + (int64_t)j * D)[c];
  }
}

// Seed scoring: every row against every seed key (dense [n_seeds, D] tile
// source) with the shared micro-kernel; grid (row groups, seed chunks of
// kSeedChunk), so that a few thousand rows still fill every CU.  The STATS
// build (grid: row groups) instead takes the per-head activation statistics
// of its rows over the 128-seed sample (dense [n_sample, D]): the count of
// x_h > 0 and the sum of max(x_h, 0); apart, the scoring build keeps the
// register budget of the plain score kernel.
constexpr int kSeedChunk = 4096;
template <int MT, int KS, int QPW, bool STATS>
__global__ __launch_bounds__(256, 2) void dosa_seed_score(
    const DosaCtx* ctx, const uint16_t* __restrict__ q, const uint16_t* __restrict__ sk,
    const uint16_t* __restrict__ smp, int n_sample, const float* __restrict__ w,
    int64_t w_stride, int n_q, int H, int n_seeds, float* __restrict__ seed_scores,
    int32_t* __restrict__ stat_cnt, float* __restrict__ stat_sum) {
  constexpr int D = 16 * KS;
  constexpr int ROWB = D * 2 + 16;
  constexpr int CPK = D * 2 / 16;
  constexpr int CHUNKS = 32 * CPK;
  constexpr int CPT = (CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][32 * ROWB];
  // this workgroup's seeds: chunk blockIdx.y of kSeedChunk
  const int s_lo = (int)blockIdx.y * kSeedChunk;
  const int s_n = n_seeds - s_lo < kSeedChunk ? n_seeds - s_lo : kSeedChunk;
  if (ctx->global_fallback) {  // rows take the exact path; keep the buffer defined
    if (!STATS)
      for (int i = 0; i < 4 * QPW; ++i) {
        const int r = (int)blockIdx.x * 4 * QPW + i;
        if (r < n_q)
          for (int j = threadIdx.x; j < s_n; j += 256)
            seed_scores[(int64_t)r * n_seeds + s_lo + j] = 0.0f;
      }
    return;
  }
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int r0 = (int)blockIdx.x * 4 * QPW + wave * QPW;

  bf16x8 a[QPW][MT][KS];
  float wv[QPW][MT][16];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    load_q_frag<MT, KS>(q, r0 + i, H, r0 + i < n_q, a[i]);
    load_w_frag<MT>(w, w_stride, r0 + i, H, r0 + i < n_q, wv[i]);
  }
  static_assert(CHUNKS % 256 == 0, "every thread stages whole chunks");
  u32x4 pre[CPT];
  // 32-key tiles of a dense key array through a buffer resource (zero past
  // its n keys, no branch around a load), double buffered in LDS; body(t,
  // brow) consumes tile t of the key array
  auto stream = [&](const uint16_t* keys, int n, auto body) {
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)keys, (short)0, n * D * 2, 0x00020000);
    auto fetch = [&](int t) {
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        pre[c] = __builtin_amdgcn_raw_buffer_load_b128(
            krs, t * (32 * D * 2) + ((int)threadIdx.x + 256 * c) * 16, 0, 0);
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        int ch = threadIdx.x + 256 * c;
        int key = ch / CPK, part = ch % CPK;
        *reinterpret_cast<u32x4*>(&lds[buf][key * ROWB + part * 16]) = pre[c];
      }
    };
    const int ntiles = (n + 31) / 32;
    __syncthreads();  // the buffers' previous contents are consumed
    fetch(0);
    stash(0);
    wait_memory();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      fetch(t + 1 < ntiles ? t + 1 : t);  // the last one is a harmless repeat
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
      body(t, &lds[buf][(lane & 31) * ROWB + (lane >> 5) * 16]);
      // buffer buf ^ 1 held tile t - 1, read before the previous barrier
      stash(buf ^ 1);
      __syncthreads();
    }
  };

  if constexpr (STATS) {  // activation statistics over the sample (padding
                         // keys are zero: x = 0 adds nothing to either statistic)
    int cnt[QPW][MT][16];
    float rs[QPW][MT][16];
#pragma unroll
    for (int i = 0; i < QPW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          cnt[i][mt][v] = 0;
          rs[i][mt][v] = 0.0f;
        }
    stream(smp, n_sample, [&](int t, const unsigned char* brow) {
      (void)t;
      f32x16 acc[QPW][MT];
      mfma_tiles<QPW, MT, KS>(
          a, [&](int s) { return as_bf16x8(*reinterpret_cast<const u32x4*>(brow + 32 * s)); },
          acc);
#pragma unroll
      for (int i = 0; i < QPW; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float x = relu(acc[i][mt][v]);
            cnt[i][mt][v] += x > 0.0f ? 1 : 0;
            rs[i][mt][v] += x;
          }
    });
    // reduce over the 32 key lanes of each half-wave
#pragma unroll
    for (int i = 0; i < QPW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int c = cnt[i][mt][v];
          float f = rs[i][mt][v];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) {
            c += __shfl_xor(c, o, 64);
            f += __shfl_xor(f, o, 64);
          }
          int h = mt * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if ((lane & 31) == 0 && r0 + i < n_q && h < H) {
            stat_cnt[(int64_t)(r0 + i) * H + h] = c;
            stat_sum[(int64_t)(r0 + i) * H + h] = f;
          }
        }
  }
  if constexpr (!STATS)
  stream(sk + (int64_t)s_lo * D, s_n, [&](int t, const unsigned char* brow) {
    f32x16 acc[QPW][MT];
    mfma_tiles<QPW, MT, KS>(
        a, [&](int s) { return as_bf16x8(*reinterpret_cast<const u32x4*>(brow + 32 * s)); },
        acc);
    const int j = t * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const float sc = head_reduce<MT>(acc[i], wv[i]);
      if (lane < 32 && r0 + i < n_q && j < s_n)
        seed_scores[(int64_t)(r0 + i) * n_seeds + s_lo + j] = sc;
    }
  });
}

__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  float f = (float)x;  // the f32 rounding is exact for the bf16 grid's decision below
  uint32_t u = __float_as_uint(f);
  // round the f32 to bf16 by nearest-even on the exact double: compare the
  // two bf16 neighbours of x directly
  uint32_t lo = u & 0xFFFF0000u;
  float flo = __uint_as_float(lo);
  float fhi = __uint_as_float(lo + 0x10000u);
  double dlo = fabs(x - (double)flo), dhi = fabs(x - (double)fhi);
  // for negative x, lo is the larger magnitude neighbour toward zero
  uint32_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = lo + 0x10000u;
  else pick = ((lo >> 16) & 1u) ? lo + 0x10000u : lo;
  return (uint16_t)(pick >> 16);
}

// Per-row plan (fp64).  One workgroup per row.  q_h rows sit in LDS as
// floats (bf16 values are exact there), 16-byte aligned.  Every per-head sum
// over d is split over TPH threads of the head (chunks of D / TPH, each
// summed in increasing d) and combined by a fixed butterfly, so the row's
// plan is the same bits on every run; no order matters for soundness, which
// the 2^-10 margin in C_r carries.
constexpr int kPlanThreads = 256;
constexpr int kPlanStride = 128 + 4;  // floats per q_h row in LDS
__device__ __forceinline__ double sum_lanes(double x, int width) {
  for (int o = 1; o < width; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__global__ __launch_bounds__(kPlanThreads) void dosa_plan(
    const DosaCtx* ctx, const uint16_t* __restrict__ q, const float* __restrict__ w,
    int64_t w_stride, int H, int D, int n_stat, int kept_heads, float neg_frac,
    const int32_t* __restrict__ stat_cnt, const float* __restrict__ stat_sum,
    uint16_t* __restrict__ plan_a, float* __restrict__ plan_w, float* __restrict__ plan_c) {
  __shared__ __attribute__((aligned(16))) float qf[64 * kPlanStride];
  __shared__ double gdot[64][32];  // q_h . q_j for omitted positive h, kept index t
  __shared__ double qq[64], wf[64], dn[64], beta[64], agg[128], part[2][128];
  __shared__ float imp[64], wrow[64];
  __shared__ int role[64], anchor[64], kept_list[32], pos_list[64];
  __shared__ int n_kept, n_pos;
  __shared__ double fin[5];
  if (ctx->global_fallback) return;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  // TPH threads per head (H <= 64): head tid / TPH, d chunk tid % TPH
  const int TPH = H <= 16 ? 16 : (H <= 32 ? 8 : 4);
  const int hh = tid / TPH, cc = tid % TPH, dlen = D / TPH, d0 = cc * dlen;
  for (int e = tid; e < H * D; e += kPlanThreads)
    qf[(e / D) * kPlanStride + e % D] = __uint_as_float((uint32_t)q[(int64_t)r * H * D + e] << 16);
  for (int h = tid; h < H; h += kPlanThreads) {
    wrow[h] = w[(int64_t)r * w_stride + h];
    imp[h] = fabsf(wrow[h]) * (stat_sum[(int64_t)r * H + h] / (float)n_stat);
  }
  __syncthreads();
  const float* qh_ = &qf[hh * kPlanStride];
  {  // |q_h|^2
    double s0 = 0.0, s1 = 0.0;
    for (int d = d0; d < d0 + dlen; d += 2) {
      const double x0 = qh_[d], x1 = qh_[d + 1];
      s0 += x0 * x0;
      s1 += x1 * x1;
    }
    const double s = sum_lanes(s0 + s1, TPH);
    if (cc == 0 && hh < H) qq[hh] = s;
  }
  if (tid < H) {
    int h = tid, rank = 0;
    for (int g = 0; g < H; ++g)
      rank += (imp[g] > imp[h] || (imp[g] == imp[h] && g < h)) ? 1 : 0;
    const float wh = wrow[h];
    const float act = (float)stat_cnt[(int64_t)r * H + h] / (float)n_stat;
    role[h] = rank < kept_heads ? 1 : (wh > 0.0f ? 2 : (wh < 0.0f ? (act >= neg_frac ? 3 : 4) : 0));
  }
  __syncthreads();
  if (tid < 64) {  // kept heads and omitted positive heads, ascending
    const bool kept = lane < H && role[lane] == 1, pos = lane < H && role[lane] == 2;
    const uint64_t km = __ballot(kept), pm = __ballot(pos);
    const uint64_t below = (1ull << lane) - 1ull;
    if (kept) kept_list[__popcll(km & below)] = lane;
    if (pos) pos_list[__popcll(pm & below)] = lane;
    if (lane == 0) {
      n_kept = __popcll(km);
      n_pos = __popcll(pm);
    }
  }
  __syncthreads();
  const int nk = n_kept, np = n_pos;
  // q_h . q_j for every omitted positive head h and kept head j
  for (int e = tid; e < np * nk; e += kPlanThreads) {
    const int h = pos_list[e / nk], j = kept_list[e % nk];
    const float4* a4 = reinterpret_cast<const float4*>(&qf[h * kPlanStride]);
    const float4* b4 = reinterpret_cast<const float4*>(&qf[j * kPlanStride]);
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    for (int d = 0; d < D / 4; ++d) {
      const float4 x = a4[d], y = b4[d];
      s0 += (double)x.x * (double)y.x;
      s1 += (double)x.y * (double)y.y;
      s2 += (double)x.z * (double)y.z;
      s3 += (double)x.w * (double)y.w;
    }
    gdot[h][e % nk] = (s0 + s1) + (s2 + s3);
  }
  __syncthreads();
  // anchor of each omitted positive head: the kept head of smallest
  // residual under the clamped projection, the lower head on ties
  if (tid < H) {
    const int h = tid;
    anchor[h] = -1;
    beta[h] = 0.0;
    if (role[h] == 2) {
      double best = INFINITY, bb = 0.0;
      int bj = -1;
      for (int t = 0; t < nk; ++t) {
        const int j = kept_list[t];
        const double g = gdot[h][t];
        double bt = qq[j] > 0.0 ? g / qq[j] : 0.0;
        bt = bt < 0.0 ? 0.0 : bt;
        const double r2 = qq[h] - 2.0 * bt * g + bt * bt * qq[j];
        if (r2 < best) {
          best = r2;
          bb = bt;
          bj = j;
        }
      }
      anchor[h] = bj;
      beta[h] = bb;
    }
  }
  __syncthreads();
  {  // |q_h - beta q_a| taken explicitly (no cancellation in the bound)
    const int a = hh < H ? anchor[hh] : -1;
    const double bb = hh < H ? beta[hh] : 0.0;
    double s0 = 0.0, s1 = 0.0;
    if (hh < H && role[hh] == 2) {
      const float* qa = &qf[(a >= 0 ? a : 0) * kPlanStride];
      for (int d = d0; d < d0 + dlen; d += 2) {
        const double e0 = (double)qh_[d] - (a >= 0 ? bb * (double)qa[d] : 0.0);
        const double e1 = (double)qh_[d + 1] - (a >= 0 ? bb * (double)qa[d + 1] : 0.0);
        s0 += e0 * e0;
        s1 += e1 * e1;
      }
    }
    const double s = sum_lanes(s0 + s1, TPH);
    if (cc == 0 && hh < H) dn[hh] = role[hh] == 2 ? sqrt(s) : 0.0;
  }
  if (tid < H) {
    const int j = tid;
    double f = 0.0;
    if (role[j] == 1) {
      f = (double)wrow[j];
      for (int h = 0; h < H; ++h)
        if (role[h] == 2 && anchor[h] == j) f += (double)wrow[h] * beta[h];
    }
    wf[j] = f;
  }
  for (int d = tid; d < D; d += kPlanThreads) {
    double s = 0.0;
    for (int h = 0; h < H; ++h)
      if (role[h] == 3) s += fabs((double)wrow[h]) * (double)qf[h * kPlanStride + d];
    agg[d] = s;
    // the aggregate's bf16 carrier and its rounding error, per d
    const double ah = (double)__uint_as_float((uint32_t)f64_to_bf16_rne(s) << 16);
    part[0][d] = (s - ah) * (s - ah);
    part[1][d] = ah * ah;
  }
  __syncthreads();
  uint16_t* pa = plan_a + (int64_t)r * 32 * D;
  for (int e = tid; e < 32 * D; e += kPlanThreads) {
    int row = e / D, d = e % D;
    uint16_t v = 0;
    if (row < nk) v = q[((int64_t)r * H + kept_list[row]) * D + d];
    else if (row == nk) v = f64_to_bf16_rne(agg[d]);
    pa[e] = v;
  }
  if (tid < 32) {
    float v = 0.0f;
    if (tid < nk) v = (float)wf[kept_list[tid]];
    else if (tid == nk) v = -1.0f;
    plan_w[(int64_t)r * 32 + tid] = v;
  }
  // the margin scalar's sums: over heads in wave 0, over d in wave 1
  if (tid < 64) {
    const int h = lane;
    double nw = 0.0, R = 0.0, nwf = 0.0;
    if (h < H) {
      const double wh = (double)wrow[h], n = sqrt(qq[h]);
      nw = fabs(wh) * n;
      R = role[h] == 2 ? wh * dn[h] : 0.0;
      nwf = role[h] == 1 ? fabs(wf[h]) * n : 0.0;
    }
    nw = sum_lanes(nw, 64);
    R = sum_lanes(R, 64);
    nwf = sum_lanes(nwf, 64);
    if (lane == 0) {
      fin[0] = nw;
      fin[1] = R;
      fin[2] = nwf;
    }
  } else if (tid < 128) {
    double e2 = 0.0, a2 = 0.0;
    for (int d = lane; d < D; d += 64) {
      e2 += part[0][d];
      a2 += part[1][d];
    }
    e2 = sum_lanes(e2, 64);
    a2 = sum_lanes(a2, 64);
    if (lane == 0) {
      fin[3] = e2;
      fin[4] = a2;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const double nw = fin[0], R = fin[1], nwf = fin[2];
    const double err = sqrt(fin[3]), ahn = sqrt(fin[4]);
    double C = R + err + 0x1p-10 * (nw + nwf + ahn + R + err);
    plan_c[r] = __double2float_ru(C);
  }
}

__global__ void dosa_knorm(const uint16_t* k, int64_t n_k, int D, float* knorm) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_k;
       j += (int64_t)gridDim.x * blockDim.x) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) {
      double x = (double)__uint_as_float((uint32_t)k[j * D + d] << 16);
      s += x * x;
    }
    knorm[j] = __double2float_ru(sqrt(s) * (1.0 + 0x1p-40));
  }
}

// Bound scan: MFMA over the 32-row plan tile of QPW rows per wave, shared
// key tiles through LDS; writes one 32-bit survivor mask per (row, tile).
// One workgroup per 4 QPW rows and key segment (score_micro.hpp).
template <int KS, int QPW>
__global__ __launch_bounds__(256, 2) void dosa_bound(
    const DosaCtx* ctx, const uint16_t* __restrict__ plan_a, const float* __restrict__ plan_w,
    const float* __restrict__ plan_c, const float* __restrict__ top_score, int topk,
    const uint16_t* __restrict__ k, const float* __restrict__ knorm,
    const uint32_t* __restrict__ seed_mask, const int32_t* __restrict__ vis_len, int n_q,
    int64_t n_k, uint32_t* __restrict__ bitmap, int64_t words, int nseg, int64_t seg_keys,
    int32_t* __restrict__ bound_cnt, int cap) {
  constexpr int D = 16 * KS;
  constexpr int QB = 4 * QPW;
  constexpr int ROWB = D * 2 + 16;
  constexpr int CPK = D * 2 / 16;
  constexpr int CHUNKS = 32 * CPK;
  constexpr int CPT = (CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][32 * ROWB];
  __shared__ int wdone[2][4];  // per tile parity: the wave has nothing left to scan
  if (ctx->global_fallback) return;
  const int lane = threadIdx.x & 63, wave = wave_index();
  int g;
  int64_t key_lo, key_hi;
  if (!segment_of((n_q + QB - 1) / QB, nseg, seg_keys, n_k, true, &g, &key_lo, &key_hi)) return;
  const int r0 = g * QB;
  int64_t vis[QPW];
  float tau[QPW], cr[QPW];
  int64_t end = 0;
  for (int i = 0; i < QB; ++i) {
    int r = r0 + i;
    int64_t off, v = 0;
    if (r < n_q) v = visible_len(vis_len, nullptr, r, n_k, n_k, &off);
    end = v > end ? v : end;
    if (i / QPW == wave) {
      vis[i % QPW] = v;
      tau[i % QPW] = r < n_q ? top_score[(int64_t)r * topk + topk - 1] : 0.0f;
      cr[i % QPW] = r < n_q ? plan_c[r] : 0.0f;
    }
  }
  end = end < key_hi ? end : key_hi;
  if (end <= key_lo) return;
  bf16x8 a[QPW][1][KS];
  float wv[QPW][1][16];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    int r = r0 + wave * QPW + i;
    load_q_frag<1, KS>(plan_a, r, 32, r < n_q, a[i]);
    load_w_frag<1>(plan_w, 32, r, 32, r < n_q, wv[i]);
  }
  const int t_lo = (int)(key_lo / 32), ntiles = (int)((end + 31) / 32);
  static_assert(CHUNKS % 256 == 0, "every thread stages whole chunks");
  // keys, norms and seed words through buffer resources (zero past n_k, no
  // branch around a load; n_k * D * 2 < 2^31 is checked by the caller)
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)k, (short)0, (int)(n_k * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t nrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)knorm, (short)0, (int)(n_k * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)seed_mask, (short)0, (int)(((n_k + 31) / 32) * 4), 0x00020000);
  u32x4 pre[CPT];
  auto fetch = [&](int t) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      pre[c] = __builtin_amdgcn_raw_buffer_load_b128(
          krs, t * (32 * D * 2) + ((int)threadIdx.x + 256 * c) * 16, 0, 0);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      int ch = threadIdx.x + 256 * c;
      int key = ch / CPK, part = ch % CPK;
      *reinterpret_cast<u32x4*>(&lds[buf][key * ROWB + part * 16]) = pre[c];
    }
  };
  // a key's norm and seed word travel one tile ahead of their use, with the
  // key tile itself
  auto side = [&](int t, float& kn, uint32_t& sw) {
    kn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                       nrs, (t * 32 + (lane & 31)) * 4, 0, 0));
    sw = __builtin_amdgcn_raw_buffer_load_b32(mrs, t * 4, 0, 0);
  };
  // Survivor counts of the wave's rows: the count of every workgroup that
  // scans them, in bound_cnt (read at the start and every kFlush tiles, past
  // the L1), plus this wave's own since its last flush.  A row with more
  // survivors than the capacity takes the exact path (its compaction reads
  // the count, not the bitmap), so its remaining tiles need no bound; once
  // no row of the workgroup needs one, the scan ends.  Every survivor is
  // flushed into bound_cnt before the workgroup ends.
  constexpr int kFlush = 16;
  int seen[QPW], mine[QPW];
  auto refresh = [&]() {
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int r = r0 + wave * QPW + i;
      seen[i] = r < n_q ? __hip_atomic_load(&bound_cnt[r], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : 0;
    }
  };
  auto flush = [&]() {
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int r = r0 + wave * QPW + i;
      if (lane == 0 && r < n_q && mine[i] > 0) atomicAdd(&bound_cnt[r], mine[i]);
      mine[i] = 0;
    }
  };
#pragma unroll
  for (int i = 0; i < QPW; ++i) mine[i] = 0;
  float kn_n;
  uint32_t sw_n;
  fetch(t_lo);
  side(t_lo, kn_n, sw_n);
  refresh();
  stash(t_lo & 1);
  wait_memory();
  __syncthreads();
  for (int t = t_lo; t < ntiles; ++t) {
    const int buf = t & 1;
    const float kn = kn_n;
    const uint32_t sw = sw_n;
    const int tn = t + 1 < ntiles ? t + 1 : t;  // the last one is a harmless repeat
    fetch(tn);
    side(tn, kn_n, sw_n);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMAs
    const int64_t j = (int64_t)t * 32 + (lane & 31);
    bool done = true;  // (uniform) no row of this wave needs this tile or a later one
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int r = r0 + wave * QPW + i;
      done = done && (r >= n_q || (int64_t)t * 32 >= vis[i] || seen[i] + mine[i] > cap);
    }
    if (done) {
      // nothing to scan for this wave's rows
    } else if (sw == 0xFFFFFFFFu) {
      // every key of the tile is a seed (the cold prior's low-index keys
      // mostly are): nothing survives, no bound to compute
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        const int r = r0 + wave * QPW + i;
        if (lane == 0 && r < n_q && (int64_t)t * 32 < vis[i]) bitmap[(int64_t)r * words + t] = 0u;
      }
    } else {
      const unsigned char* brow = &lds[buf][(lane & 31) * ROWB + (lane >> 5) * 16];
      f32x16 acc[QPW][1];
      mfma_tiles<QPW, 1, KS>(
          a, [&](int s) { return as_bf16x8(*reinterpret_cast<const u32x4*>(brow + 32 * s)); },
          acc);
      const bool seed = (sw >> (j & 31)) & 1u;
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        float u = head_reduce<1>(acc[i], wv[i]) + cr[i] * kn;
        bool pass = lane < 32 && j < vis[i] && !seed && u >= tau[i];
        uint64_t m = __ballot(pass);
        int r = r0 + wave * QPW + i;
        if (lane == 0 && r < n_q && (int64_t)t * 32 < vis[i])
          bitmap[(int64_t)r * words + t] = (uint32_t)m;
        mine[i] += __popcll(m);
      }
    }
    if (lane == 0) wdone[buf][wave] = done ? 1 : 0;
    if ((t - t_lo) % kFlush == kFlush - 1) {
      flush();
      refresh();
    }
    // buffer buf ^ 1 held tile t - 1, read before the previous barrier
    stash(buf ^ 1);
    __syncthreads();
    // (wdone[buf] is rewritten two tiles on, after every wave has passed
    // the next barrier and so has read it here)
    if (wdone[buf][0] & wdone[buf][1] & wdone[buf][2] & wdone[buf][3]) break;
  }
  flush();
}

// Bitmap -> ascending survivor ids (one workgroup per row).
constexpr int kCompThreads = 256;
constexpr int kCompStage = 8192;  // ids a round stages in LDS (capacities up to this)
__global__ __launch_bounds__(kCompThreads) void dosa_compact(
    const DosaCtx* ctx, const uint32_t* __restrict__ bitmap, int64_t words,
    const int32_t* __restrict__ vis_len, int64_t n_k, int cap, const int32_t* __restrict__ bound_cnt,
    int32_t* __restrict__ surv_ids, int32_t* __restrict__ surv_cnt, int32_t* __restrict__ row_fb) {
  __shared__ int red[kCompThreads / 64 + 4];
  const int r = blockIdx.x;
  if (ctx->global_fallback) {
    if (threadIdx.x == 0) {
      surv_cnt[r] = 0;
      row_fb[r] = 1;
    }
    return;
  }
  // a row over the capacity may have tiles the bound scan skipped: its
  // count decides, and its bitmap is not read
  const int counted = bound_cnt[r];
  const bool over = counted > cap;
  int64_t off;
  const int64_t v = visible_len(vis_len, nullptr, r, n_k, n_k, &off);
  const int64_t nw = over ? 0 : (v + 31) / 32;
  const uint32_t* brow = bitmap + (int64_t)r * words;
  int32_t* out = surv_ids + (int64_t)r * cap;
  int total = 0;
  if (cap <= kCompStage) {
    // rounds of 4 kCompThreads words, thread t taking words 4t .. 4t + 3:
    // a block scan of the per-thread counts places each id in LDS, and the
    // round's ids leave in one coalesced pass (a round never holds more than
    // the row's count, at most cap <= kCompStage)
    __shared__ int32_t stage[kCompStage];
    const int t = (int)threadIdx.x;
    for (int64_t r0 = 0; r0 < nw; r0 += 4 * kCompThreads) {
      const int64_t wi = r0 + 4 * t;
      uint32_t m[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) m[j] = wi + j < nw ? brow[wi + j] : 0u;
      const int c = __popc(m[0]) + __popc(m[1]) + __popc(m[2]) + __popc(m[3]);
      int tot;
      int p = block_excl_scan<kCompThreads>(c, red, &tot);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        for (uint32_t mm = m[j]; mm != 0u; mm &= mm - 1u) {
          if (p < kCompStage) stage[p] = (int32_t)((wi + j) * 32 + (__ffs(mm) - 1));
          ++p;
        }
      __syncthreads();
      for (int i = t; i < tot && i < kCompStage; i += kCompThreads)
        if (total + i < cap) out[total + i] = stage[i];
      total += tot;
      __syncthreads();  // the next round's ids reuse the stage
    }
  } else {
    const int64_t per = (nw + kCompThreads - 1) / kCompThreads;
    const int64_t w0 = (int64_t)threadIdx.x * per;
    int mine = 0;
    for (int64_t i = w0; i < w0 + per && i < nw; ++i) mine += __popc(brow[i]);
    int pos = block_excl_scan<kCompThreads>(mine, red, &total);
    for (int64_t i = w0; i < w0 + per && i < nw; ++i) {
      uint32_t m = brow[i];
      while (m) {
        int b = __ffs(m) - 1;
        m &= m - 1;
        out[pos++] = (int32_t)(i * 32 + b);
      }
    }
  }
  if (threadIdx.x == 0) {
    surv_cnt[r] = over ? counted : total;
    row_fb[r] = over ? 1 : 0;
  }
}

// Slot of this lane's item in a list whose length is *cnt, for the lanes
// with keep set: one atomic per wave (every lane of the wave calls it).
__device__ __forceinline__ int wave_append(bool keep, int32_t* cnt) {
  const uint64_t m = __ballot(keep);
  int base = 0;
  if ((threadIdx.x & 63) == 0 && m) base = atomicAdd(cnt, __popcll(m));
  base = __shfl(base, 0);
  return base + __popcll(m & ((1ull << (threadIdx.x & 63)) - 1ull));
}

// Exact rescoring of survivors with the shared micro-kernel (keys gathered
// straight into the k-step layout, one tile ahead).  One workgroup per row.
template <int MT, int KS>
__global__ __launch_bounds__(256) void dosa_rescore(
    const DosaCtx* ctx, const uint16_t* __restrict__ q, const float* __restrict__ w,
    int64_t w_stride, int H, const uint16_t* __restrict__ k, const float* __restrict__ top_score,
    int topk, const int32_t* __restrict__ surv_ids, const int32_t* __restrict__ list_cnt,
    const int32_t* __restrict__ row_fb, int cap, float* __restrict__ kept_score,
    int32_t* __restrict__ kept_id, int32_t* __restrict__ kept_cnt) {
  constexpr int D = 16 * KS;
  const int r = blockIdx.x;
  if (ctx->global_fallback || row_fb[r]) return;
  const int n = list_cnt[r];
  if (n == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float tau = top_score[(int64_t)r * topk + topk - 1];
  bf16x8 a[1][MT][KS];
  float wv[MT][16];
  load_q_frag<MT, KS>(q, r, H, true, a[0]);
  load_w_frag<MT>(w, w_stride, r, H, true, wv);
  // tiles wave * 32 + 128 i; the next tile's ids are read and its keys
  // gathered into registers during this tile's MFMAs
  auto gather = [&](int t0, int& id, u32x4 (&kb)[KS]) {
    const int i = t0 + (lane & 31);
    id = i < n ? surv_ids[(int64_t)r * cap + i] : -1;
    const u32x4* src = reinterpret_cast<const u32x4*>(k + (int64_t)(id >= 0 ? id : 0) * D);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kb[s] = id >= 0 ? src[2 * s + (lane >> 5)] : u32x4{0u, 0u, 0u, 0u};
  };
  int id_c = -1, id_n = -1;
  u32x4 kc[KS], kn[KS];
  if (wave * 32 < n) gather(wave * 32, id_c, kc);
  for (int t0 = wave * 32; t0 < n; t0 += 4 * 32) {
    if (t0 + 128 < n) gather(t0 + 128, id_n, kn);
    f32x16 acc[1][MT];
    mfma_tiles<1, MT, KS>(a, [&](int s) { return as_bf16x8(kc[s]); }, acc);
    float s = head_reduce<MT>(acc[0], wv);
    const bool keep = lane < 32 && id_c >= 0 && s >= tau;
    const int slot = wave_append(keep, &kept_cnt[r]);
    if (keep) {
      kept_score[(int64_t)r * cap + slot] = s;
      kept_id[(int64_t)r * cap + slot] = id_c;
    }
    id_c = id_n;
#pragma unroll
    for (int j = 0; j < KS; ++j) kc[j] = kn[j];
  }
}

// 4-query groups (one workgroup per group).  A row whose survivors (keys
// passing its bound) exceed the capacity takes the exact path, as with
// per-row streams, and its bits take no part in the split.  Of the other
// rows' survivors, a key set for at least 2 of them and below the group's
// common visible prefix goes to the shared stream, every other one to its
// row's solo stream, both ascending.  A shared key is set for at least two
// rows of at most the capacity each, so the shared stream holds at most
// 2 * capacity keys, and a row keeps at most its own survivors.  surv_cnt
// keeps each row's survivor count, shared_n the part the shared stream
// carries.
constexpr int kGroupRows = 4;
__global__ __launch_bounds__(kCompThreads) void dosa_compact_groups(
    const DosaCtx* ctx, const uint32_t* __restrict__ bitmap, int64_t words,
    const int32_t* __restrict__ vis_len, int n_q, int64_t n_k, int cap,
    const int32_t* __restrict__ bound_cnt,
    int32_t* __restrict__ shared_ids, int32_t* __restrict__ shared_cnt,
    int32_t* __restrict__ surv_ids, int32_t* __restrict__ solo_cnt,
    int32_t* __restrict__ surv_cnt, int32_t* __restrict__ shared_n, int32_t* __restrict__ row_fb) {
  __shared__ int red[kCompThreads / 64 + 4];
  const int g = blockIdx.x, t = threadIdx.x;
  const int r0 = g * kGroupRows;
  const int nr = n_q - r0 < kGroupRows ? n_q - r0 : kGroupRows;
  if (ctx->global_fallback) {
    if (t < nr) {
      surv_cnt[r0 + t] = 0;
      solo_cnt[r0 + t] = 0;
      shared_n[r0 + t] = 0;
      row_fb[r0 + t] = 1;
    }
    if (t == 0) shared_cnt[g] = 0;
    return;
  }
  int64_t nwr[kGroupRows];
  int64_t cg = INT64_MAX, nw = 0;
#pragma unroll
  for (int i = 0; i < kGroupRows; ++i) {
    int64_t off, v = 0;
    if (i < nr) v = visible_len(vis_len, nullptr, r0 + i, n_k, n_k, &off);
    nwr[i] = (v + 31) / 32;
    if (i < nr) cg = v < cg ? v : cg;
    nw = nwr[i] > nw ? nwr[i] : nw;
  }
  const int64_t per = (nw + kCompThreads - 1) / kCompThreads;
  const int64_t w0 = (int64_t)t * per;
  // each row's survivors; a row over the capacity (its count, which may
  // miss tiles the bound scan skipped, decides) takes the exact path and
  // its bitmap is not read
  bool over[kGroupRows];
  int counted[kGroupRows];
#pragma unroll
  for (int i = 0; i < kGroupRows; ++i) {
    counted[i] = i < nr ? bound_cnt[r0 + i] : 0;
    over[i] = counted[i] > cap;
  }
  int tot[kGroupRows] = {0, 0, 0, 0}, tot_total[kGroupRows];
  for (int64_t wi = w0; wi < w0 + per && wi < nw; ++wi)
#pragma unroll
    for (int i = 0; i < kGroupRows; ++i)
      if (!over[i] && wi < nwr[i]) tot[i] += __popc(bitmap[(int64_t)(r0 + i) * words + wi]);
#pragma unroll
  for (int i = 0; i < kGroupRows; ++i) (void)block_excl_scan<kCompThreads>(tot[i], red, &tot_total[i]);
  // the word's masks (rows taking the exact path contribute none), and the
  // shared part
  auto masks = [&](int64_t wi, uint32_t (&m)[kGroupRows]) -> uint32_t {
#pragma unroll
    for (int i = 0; i < kGroupRows; ++i)
      m[i] = (!over[i] && wi < nwr[i]) ? bitmap[(int64_t)(r0 + i) * words + wi] : 0u;
    const uint32_t two = (m[0] & m[1]) | (m[0] & m[2]) | (m[0] & m[3]) | (m[1] & m[2]) |
                         (m[1] & m[3]) | (m[2] & m[3]);
    const int64_t lo = wi * 32;
    const uint32_t common = lo + 32 <= cg ? 0xFFFFFFFFu
                            : (lo >= cg ? 0u : ((1u << (uint32_t)(cg - lo)) - 1u));
    return two & common;
  };
  int sh = 0, so[kGroupRows] = {0, 0, 0, 0};
  for (int64_t wi = w0; wi < w0 + per && wi < nw; ++wi) {
    uint32_t m[kGroupRows];
    const uint32_t sm = masks(wi, m);
    sh += __popc(sm);
#pragma unroll
    for (int i = 0; i < kGroupRows; ++i) so[i] += __popc(m[i] & ~sm);
  }
  int sh_total, so_total[kGroupRows], spos[kGroupRows];
  int pos = block_excl_scan<kCompThreads>(sh, red, &sh_total);
#pragma unroll
  for (int i = 0; i < kGroupRows; ++i) spos[i] = block_excl_scan<kCompThreads>(so[i], red, &so_total[i]);
  for (int64_t wi = w0; wi < w0 + per && wi < nw; ++wi) {
    uint32_t m[kGroupRows];
    const uint32_t sm = masks(wi, m);
    for (uint32_t b = sm; b; b &= b - 1)
      shared_ids[(int64_t)g * 2 * cap + pos++] = (int32_t)(wi * 32 + __ffs(b) - 1);
#pragma unroll
    for (int i = 0; i < kGroupRows; ++i)
      for (uint32_t b = m[i] & ~sm; b; b &= b - 1)
        surv_ids[(int64_t)(r0 + i) * cap + spos[i]++] = (int32_t)(wi * 32 + __ffs(b) - 1);
  }
  if (t == 0) shared_cnt[g] = sh_total;
  if (t < nr) {
    surv_cnt[r0 + t] = over[t] ? counted[t] : tot_total[t];
    solo_cnt[r0 + t] = over[t] ? 0 : so_total[t];
    shared_n[r0 + t] = over[t] ? 0 : tot_total[t] - so_total[t];
    row_fb[r0 + t] = over[t] ? 1 : 0;
  }
}

// A group's shared stream: each 32-key tile is staged once in LDS (rows
// padded to 2 D + 16 bytes, so the k-step reads of 32 keys hit distinct
// banks) and scored by the group's four waves, one per row, with the shared
// micro-kernel; a row keeps the keys with s >= its tau.  Two LDS tiles
// alternate: the next tile's keys are loaded into registers during this
// tile's MFMAs (their ids one tile earlier still) and stored into the other
// tile, whose last reads the previous iteration's barrier has retired.
// Grid (groups, kSharedSplit): workgroup (g, y) takes the y-th run of the
// stream's 32-key tiles, so a long stream spreads over several CUs.
constexpr int kSharedSplit = 16;
template <int MT, int KS>
__global__ __launch_bounds__(256) void dosa_rescore_shared(
    const DosaCtx* ctx, const uint16_t* __restrict__ q, const float* __restrict__ w,
    int64_t w_stride, int n_q, int H, const uint16_t* __restrict__ k,
    const float* __restrict__ top_score, int topk, const int32_t* __restrict__ shared_ids,
    const int32_t* __restrict__ shared_cnt, const int32_t* __restrict__ row_fb, int cap,
    float* __restrict__ kept_score, int32_t* __restrict__ kept_id,
    int32_t* __restrict__ kept_cnt) {
  constexpr int D = 16 * KS;
  constexpr int RB = 2 * D + 16;           // LDS bytes per staged key
  constexpr int CPK = D / 8;               // 16-byte chunks per key
  constexpr int NC = (32 * CPK + 255) / 256;  // chunks per thread per tile
  __shared__ __attribute__((aligned(16))) unsigned char tile[2][32 * RB];
  const int g = blockIdx.x;
  if (ctx->global_fallback) return;
  const int n_all = shared_cnt[g];
  const int tiles = (n_all + 31) / 32;
  const int tpp = (tiles + kSharedSplit - 1) / kSharedSplit;
  const int first = (int)blockIdx.y * tpp * 32;
  if (first >= n_all) return;
  const int n = n_all - first < tpp * 32 ? n_all - first : tpp * 32;  // keys of this run
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = g * kGroupRows + wave;
  const bool active = r < n_q && !row_fb[r];
  const int rq = r < n_q ? r : n_q - 1;
  const int32_t* ids = shared_ids + (int64_t)g * 2 * cap + first;
  auto fetch_ids = [&](int t0, int (&id)[NC]) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int i = t0 + c / CPK;
      id[j] = (c < 32 * CPK && i < n) ? ids[i] : -1;
    }
  };
  auto fetch_keys = [&](const int (&id)[NC], u32x4 (&v)[NC]) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = threadIdx.x + 256 * j;
      v[j] = id[j] >= 0 ? reinterpret_cast<const u32x4*>(k + (int64_t)id[j] * D)[c % CPK]
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stash = [&](int b, const u32x4 (&v)[NC]) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = threadIdx.x + 256 * j;
      if (c < 32 * CPK) *reinterpret_cast<u32x4*>(&tile[b][(c / CPK) * RB + (c % CPK) * 16]) = v[j];
    }
  };
  int id_cur[NC], id_next[NC];
  u32x4 v[NC];
  fetch_ids(0, id_cur);
  fetch_ids(32, id_next);
  fetch_keys(id_cur, v);
  bf16x8 a[1][MT][KS];
  float wv[MT][16];
  load_q_frag<MT, KS>(q, rq, H, true, a[0]);
  load_w_frag<MT>(w, w_stride, rq, H, true, wv);
  const float tau = top_score[(int64_t)rq * topk + topk - 1];
  stash(0, v);
  __syncthreads();
  for (int it = 0; it * 32 < n; ++it) {
    const int t0 = it * 32;
    const bool more = t0 + 32 < n;
    if (more) {
      fetch_keys(id_next, v);
      fetch_ids(t0 + 64, id_next);
    }
    if (active) {
      f32x16 acc[1][MT];
      const unsigned char* kr = &tile[it & 1][(lane & 31) * RB];
      mfma_tiles<1, MT, KS>(
          a,
          [&](int s) {
            return as_bf16x8(*reinterpret_cast<const u32x4*>(kr + (2 * s + (lane >> 5)) * 16));
          },
          acc);
      const float sc = head_reduce<MT>(acc[0], wv);
      const int i = t0 + (lane & 31);
      const bool keep = lane < 32 && i < n && sc >= tau;
      const int slot = wave_append(keep, &kept_cnt[r]);
      if (keep) {
        kept_score[(int64_t)r * cap + slot] = sc;
        kept_id[(int64_t)r * cap + slot] = ids[i];
      }
    }
    if (more) stash((it + 1) & 1, v);
    __syncthreads();
  }
}

// First K of (seed top-K) u (kept survivors) by (score desc, key asc).
constexpr int kMergeThreads = 1024;
__global__ __launch_bounds__(kMergeThreads) void dosa_merge(
    const DosaCtx* ctx, const int32_t* __restrict__ row_fb, const int32_t* __restrict__ top_idx,
    const float* __restrict__ top_score, int topk, const float* __restrict__ kept_score,
    const int32_t* __restrict__ kept_id, const int32_t* __restrict__ kept_cnt, int cap,
    int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  // dynamic LDS: B [next_pow2(cap)] kept composites, then A [topk]
  extern __shared__ uint64_t merge_lds[];
  uint64_t* B = merge_lds;
  uint64_t* A = merge_lds + next_pow2(cap);
  const int r = blockIdx.x;
  if (ctx->global_fallback || row_fb[r]) return;
  const int m = kept_cnt[r];
  const int P = next_pow2(m > 1 ? m : 1);
  for (int i = threadIdx.x; i < P; i += kMergeThreads)
    B[i] = i < m ? composite(order_key(kept_score[(int64_t)r * cap + i]),
                             (uint32_t)kept_id[(int64_t)r * cap + i])
                 : 0ull;
  for (int i = threadIdx.x; i < topk; i += kMergeThreads)
    A[i] = composite(order_key(top_score[(int64_t)r * topk + i]),
                     (uint32_t)top_idx[(int64_t)r * topk + i]);
  __syncthreads();
  bitonic_sort_desc<kMergeThreads>(B, P);
  // rank in the merged order = own index + number of the other list's items
  // ranking ahead (composites are distinct: the lists hold distinct keys)
  auto count_greater = [](const uint64_t* L, int n, uint64_t x) {
    int lo = 0, hi = n;  // L descending: first index with L[i] < x
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (L[mid] > x) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  int32_t* oi = out_idx + (int64_t)r * topk;
  float* os = out_score ? out_score + (int64_t)r * topk : nullptr;
  for (int i = threadIdx.x; i < topk; i += kMergeThreads) {
    int pos = i + count_greater(B, m, A[i]);
    if (pos < topk) {
      oi[pos] = (int32_t)comp_idx(A[i]);
      if (os) os[pos] = key_to_float(comp_key(A[i]));
    }
  }
  for (int i = threadIdx.x; i < m; i += kMergeThreads) {
    int pos = i + count_greater(A, topk, B[i]);
    if (pos < topk) {
      oi[pos] = (int32_t)comp_idx(B[i]);
      if (os) os[pos] = key_to_float(comp_key(B[i]));
    }
  }
}

__global__ __launch_bounds__(1024) void dosa_fallback_list(DosaCtx* ctx, const int32_t* row_fb,
                                                           int n_q, int32_t* list) {
  __shared__ int red[1024 / 64 + 4];
  int before = 0;
  const int all = ctx->global_fallback;
  for (int base = 0; base < n_q; base += 1024) {
    int r = base + threadIdx.x;
    int f = (r < n_q && (all || row_fb[r])) ? 1 : 0;
    int tot;
    int pos = before + block_excl_scan<1024>(f, red, &tot);
    if (f) list[pos] = r;
    before += tot;
  }
  if (threadIdx.x == 0) ctx->n_fallback = before;
}

__global__ void dosa_stats(const DosaCtx* ctx, const float* top_score, int topk,
                           const int32_t* shared_n, const int32_t* surv_cnt,
                           const int32_t* row_fb, int n_q, float* tau, int32_t* n_surv,
                           int32_t* fallback, int32_t* n_shared) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < n_q; r += gridDim.x * blockDim.x) {
    const int all = ctx->global_fallback;
    if (tau) tau[r] = all ? __builtin_nanf("") : top_score[(int64_t)r * topk + topk - 1];
    if (n_surv) n_surv[r] = all ? -1 : surv_cnt[r];
    if (fallback) fallback[r] = (all || row_fb[r]) ? 1 : 0;
    if (n_shared) n_shared[r] = (all || !shared_n) ? 0 : shared_n[r];
  }
}

static unsigned grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g > 65536) g = 65536;
  return (unsigned)(g > 0 ? g : 1);
}

#define SI_TRY(expr)                                  \
  do {                                                \
    hipLaunchKernelGGL expr;                          \
    hipError_t e_ = hipGetLastError();                \
    if (e_ != hipSuccess) return e_;                  \
  } while (0)

template <int MT, int KS>
static hipError_t run_dosa(const uint16_t* q, const uint16_t* k, const float* w, int64_t wst,
                           const int32_t* vis, int n_q, int H, int64_t n_k, int topk,
                           const si_dosa_params* p, int32_t* out_idx, float* out_score,
                           const si_dosa_stats* stats, unsigned char* ws, hipStream_t st) {
  constexpr int D = 16 * KS;
  const DosaLayout L = dosa_layout(n_q, H, D, n_k, topk, p);
  DosaCtx* ctx = reinterpret_cast<DosaCtx*>(ws + L.ctx);
  auto I = [&](size_t o) { return reinterpret_cast<int32_t*>(ws + o); };
  auto F = [&](size_t o) { return reinterpret_cast<float*>(ws + o); };
  auto U16 = [&](size_t o) { return reinterpret_cast<uint16_t*>(ws + o); };
  const int R = p->n_rep_queries, ns = p->n_seeds, cap = p->survivor_capacity;
  const int64_t words = (n_k + 31) / 32;

  SI_TRY((dosa_init, dim3(1), dim3(1024), 0, st, ctx, vis, n_q, n_k, ns, I(L.rep_vis), R));
  SI_TRY((fill_i32, dim3(grid_for(n_k, 256)), dim3(256), 0, st, I(L.counts), n_k, 0));
  SI_TRY((fill_i32, dim3(grid_for(words, 256)), dim3(256), 0, st, I(L.seed_mask), words, 0));
  SI_TRY((fill_i32, dim3(grid_for(n_q, 256)), dim3(256), 0, st, I(L.kept_cnt), (int64_t)n_q, 0));
  SI_TRY((fill_i32, dim3(grid_for(n_q, 256)), dim3(256), 0, st, I(L.bound_cnt), (int64_t)n_q, 0));
  if (p->seed_ids == nullptr) {
    SI_TRY((dosa_gather_rep, dim3(R), dim3(256), 0, st, q, w, wst, n_q, H, D, R, U16(L.rep_q),
            F(L.rep_w)));
    ScoreArgs sa;
    sa.q = U16(L.rep_q); sa.q_dtype = SI_BF16; sa.k = k; sa.k_dtype = SI_BF16;
    sa.k_scale = nullptr; sa.w = F(L.rep_w); sa.w_row_stride = H; sa.k_row_offset = nullptr;
    sa.vis_len = I(L.rep_vis); sa.n_q = R; sa.H = H; sa.D = D; sa.n_k = n_k; sa.max_vis = n_k;
    sa.scores = F(L.rep_scores); sa.score_stride = n_k;
    hipError_t e = launch_score(sa, st);
    if (e != hipSuccess) return e;
    TopkArgs ta;
    ta.scores = F(L.rep_scores); ta.stride = n_k; ta.vis_len = I(L.rep_vis);
    ta.k_row_offset = nullptr; ta.n_k = n_k; ta.max_vis = n_k; ta.n_rows = R;
    ta.K = p->rep_topk; ta.out_idx = I(L.rep_ids); ta.out_score = nullptr;
    ta.workspace = ws + L.topk_ws; ta.workspace_bytes = L.topk_ws_bytes;
    e = launch_topk(ta, st);
    if (e != hipSuccess) return e;
    SI_TRY((dosa_count, dim3(grid_for((int64_t)R * p->rep_topk, 256)), dim3(256), 0, st,
            I(L.rep_ids), (int64_t)R * p->rep_topk, I(L.counts), n_k));
  }
  SI_TRY((dosa_select_seeds, dim3(1), dim3(1024), 0, st, ctx, I(L.counts), R, ns, p->seed_ids,
          I(L.seeds), reinterpret_cast<uint32_t*>(ws + L.seed_mask)));
  SI_TRY((dosa_gather_seed_keys, dim3(grid_for((int64_t)ns * (D / 8), 256)), dim3(256), 0, st,
          ctx, k, I(L.seeds), ns, D, U16(L.seed_keys)));
  SI_TRY((dosa_gather_sample, dim3(1), dim3(256), 0, st, ctx, k, I(L.seeds), ns, D,
          U16(L.sample_keys)));
  constexpr int QPW = MT == 1 ? 2 : 1;
  const int n_stat = stat_sample_size(ns);
  SI_TRY(((dosa_seed_score<MT, KS, QPW, true>), dim3((n_q + 4 * QPW - 1) / (4 * QPW)),
          dim3(256), 0, st, ctx, q, U16(L.seed_keys), U16(L.sample_keys), n_stat, w, wst, n_q, H,
          ns, F(L.seed_scores), I(L.stat_cnt), F(L.stat_sum)));
  SI_TRY(((dosa_seed_score<MT, KS, QPW, false>),
          dim3((n_q + 4 * QPW - 1) / (4 * QPW), (ns + kSeedChunk - 1) / kSeedChunk), dim3(256), 0,
          st, ctx, q, U16(L.seed_keys), U16(L.sample_keys), n_stat, w, wst, n_q, H, ns,
          F(L.seed_scores), I(L.stat_cnt), F(L.stat_sum)));
  {
    TopkArgs ta;
    ta.scores = F(L.seed_scores); ta.stride = ns; ta.vis_len = nullptr; ta.k_row_offset = nullptr;
    ta.n_k = ns; ta.max_vis = ns; ta.n_rows = n_q; ta.K = topk; ta.out_idx = I(L.top_idx);
    ta.out_score = F(L.top_score); ta.id_map = I(L.seeds);
    ta.workspace = ws + L.topk_ws; ta.workspace_bytes = L.topk_ws_bytes;
    hipError_t e = launch_topk(ta, st);
    if (e != hipSuccess) return e;
  }
  SI_TRY((dosa_plan, dim3(n_q), dim3(kPlanThreads), 0, st, ctx, q, w, wst, H, D, n_stat,
          p->kept_heads, p->neg_active_frac, I(L.stat_cnt), F(L.stat_sum), U16(L.plan_a),
          F(L.plan_w), F(L.plan_c)));
  SI_TRY((dosa_knorm, dim3(grid_for(n_k, 256)), dim3(256), 0, st, k, n_k, D, F(L.knorm)));
  {
    int64_t seg_keys;
    const int nseg = key_segments(n_k, D, &seg_keys);
    SI_TRY(((dosa_bound<KS, 2>), dim3((unsigned)segment_grid((n_q + 7) / 8, nseg)), dim3(256), 0,
            st, ctx, U16(L.plan_a), F(L.plan_w), F(L.plan_c), F(L.top_score), topk, k,
            F(L.knorm), reinterpret_cast<const uint32_t*>(ws + L.seed_mask), vis, n_q, n_k,
            reinterpret_cast<uint32_t*>(ws + L.bitmap), words, nseg, seg_keys, I(L.bound_cnt),
            cap));
  }
  const bool groups = p->shared_streams != 0;
  const int n_groups = (n_q + kGroupRows - 1) / kGroupRows;
  if (groups) {
    SI_TRY((dosa_compact_groups, dim3(n_groups), dim3(kCompThreads), 0, st, ctx,
            reinterpret_cast<const uint32_t*>(ws + L.bitmap), words, vis, n_q, n_k, cap,
            I(L.bound_cnt), I(L.shared_ids), I(L.shared_cnt), I(L.surv_ids), I(L.solo_cnt), I(L.surv_cnt),
            I(L.shared_n), I(L.row_fb)));
  } else {
    SI_TRY((dosa_compact, dim3(n_q), dim3(kCompThreads), 0, st, ctx,
            reinterpret_cast<const uint32_t*>(ws + L.bitmap), words, vis, n_k, cap,
            I(L.bound_cnt), I(L.surv_ids), I(L.surv_cnt), I(L.row_fb)));
  }
  SI_TRY(((dosa_rescore<MT, KS>), dim3(n_q), dim3(256), 0, st, ctx, q, w, wst, H, k, F(L.top_score),
          topk, I(L.surv_ids), I(groups ? L.solo_cnt : L.surv_cnt), I(L.row_fb), cap,
          F(L.kept_score), I(L.kept_id), I(L.kept_cnt)));
  if (groups)
    SI_TRY(((dosa_rescore_shared<MT, KS>), dim3(n_groups, kSharedSplit), dim3(256), 0, st, ctx,
            q, w, wst, n_q,
            H, k, F(L.top_score), topk, I(L.shared_ids), I(L.shared_cnt), I(L.row_fb), cap,
            F(L.kept_score), I(L.kept_id), I(L.kept_cnt)));
  {
    // LDS sized by the capacity and K rather than their maxima: more rows
    // per CU
    const size_t lds = (size_t)(next_pow2(cap) + topk) * sizeof(uint64_t);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dosa_merge),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  SI_TRY((dosa_merge, dim3(n_q), dim3(kMergeThreads),
          (size_t)(next_pow2(cap) + topk) * sizeof(uint64_t), st, ctx, I(L.row_fb), I(L.top_idx),
          F(L.top_score), topk, F(L.kept_score), I(L.kept_id), I(L.kept_cnt), cap, out_idx,
          out_score));
  SI_TRY((dosa_fallback_list, dim3(1), dim3(1024), 0, st, ctx, I(L.row_fb), n_q, I(L.fb_list)));
  {
    ScoreArgs sa;
    sa.q = q; sa.q_dtype = SI_BF16; sa.k = k; sa.k_dtype = SI_BF16; sa.k_scale = nullptr;
    sa.w = w; sa.w_row_stride = wst; sa.k_row_offset = nullptr; sa.vis_len = vis; sa.n_q = n_q;
    sa.H = H; sa.D = D; sa.n_k = n_k; sa.max_vis = n_k; sa.scores = F(L.fb_scores);
    sa.score_stride = n_k;
    hipError_t e = launch_score_rows_listed(sa, I(L.fb_list), &ctx->n_fallback, st);
    if (e != hipSuccess) return e;
    TopkArgs ta;
    ta.scores = F(L.fb_scores); ta.stride = n_k; ta.vis_len = vis; ta.k_row_offset = nullptr;
    ta.n_k = n_k; ta.max_vis = n_k; ta.n_rows = n_q; ta.K = topk; ta.out_idx = out_idx;
    ta.out_score = out_score; ta.row_list = I(L.fb_list); ta.row_count = &ctx->n_fallback;
    ta.workspace = ws + L.topk_ws; ta.workspace_bytes = L.topk_ws_bytes;
    e = launch_topk(ta, st);
    if (e != hipSuccess) return e;
  }
  if (stats && (stats->tau || stats->n_survivors || stats->fallback || stats->n_shared))
    SI_TRY((dosa_stats, dim3(grid_for(n_q, 256)), dim3(256), 0, st, ctx, F(L.top_score), topk,
            groups ? I(L.shared_n) : nullptr, I(L.surv_cnt), I(L.row_fb), n_q, stats->tau,
            stats->n_survivors, stats->fallback, stats->n_shared));
  return hipSuccess;
}

}  // namespace si

using namespace si;

extern "C" size_t dosa_prune_topk_workspace(int32_t n_q, int32_t H, int32_t D, int64_t n_k,
                                            int32_t topk, const si_dosa_params* p) {
  if (!p || n_q < 0 || H < 1 || D < 1 || n_k < 0 || topk < 1 || p->n_rep_queries < 1 ||
      p->n_seeds < 1 || p->rep_topk < 1 || p->survivor_capacity < 1)
    return 0;
  return dosa_layout(n_q, H, D, n_k, topk, p).total;
}

extern "C" si_status dosa_prune_topk(const void* q, const void* k, si_dtype dtype, const float* w,
                                     int64_t w_row_stride, const int32_t* vis_len, int32_t n_q,
                                     int32_t H, int32_t D, int64_t n_k, int32_t topk,
                                     const si_dosa_params* p, int32_t* out_idx, float* out_score,
                                     const si_dosa_stats* stats, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  if (!p || n_q < 0 || H < 1 || H > 64 || (D != 64 && D != 128) || n_k < 0 ||
      n_k * D * 2 > INT32_MAX || topk < 1 || topk > kMaxTopk || w_row_stride < 0)
    return SI_ERR_INVALID_ARGUMENT;
  if (p->n_seeds < topk || (int64_t)p->n_seeds > n_k || p->n_rep_queries < 1 ||
      p->n_rep_queries > kMaxRep || p->rep_topk < 1 || p->rep_topk > kMaxTopk ||
      p->kept_heads < 0 || p->kept_heads > 31 || p->kept_heads > H ||
      p->survivor_capacity < 1 || p->survivor_capacity > kMaxCapacity ||
      !(p->neg_active_frac == p->neg_active_frac) || p->shared_streams < 0 ||
      p->shared_streams > 1)
    return SI_ERR_INVALID_ARGUMENT;
  if (dtype != SI_BF16) return SI_ERR_UNSUPPORTED_DTYPE;
  if (n_q == 0) return SI_OK;
  if (!q || !k || !w || !vis_len || !out_idx) return SI_ERR_INVALID_ARGUMENT;
  auto al = [](const void* x, uintptr_t a) { return (reinterpret_cast<uintptr_t>(x) & (a - 1)) == 0; };
  if (!al(q, 16) || !al(k, 16) || !al(w, 4) || !al(out_idx, 4) || (out_score && !al(out_score, 4)) ||
      (p->seed_ids && !al(p->seed_ids, 4)))
    return SI_ERR_INVALID_ARGUMENT;
  const size_t need = dosa_layout(n_q, H, D, n_k, topk, p).total;
  if (!workspace || workspace_bytes < need || !al(workspace, 256)) return SI_ERR_WORKSPACE_TOO_SMALL;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(q);
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(k);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  hipError_t e;
  const bool mt1 = H <= 32;
  if (D == 128)
    e = mt1 ? run_dosa<1, 8>(qb, kb, w, w_row_stride, vis_len, n_q, H, n_k, topk, p, out_idx,
                             out_score, stats, ws, stream)
            : run_dosa<2, 8>(qb, kb, w, w_row_stride, vis_len, n_q, H, n_k, topk, p, out_idx,
                             out_score, stats, ws, stream);
  else
    e = mt1 ? run_dosa<1, 4>(qb, kb, w, w_row_stride, vis_len, n_q, H, n_k, topk, p, out_idx,
                             out_score, stats, ws, stream)
            : run_dosa<2, 4>(qb, kb, w, w_row_stride, vis_len, n_q, H, n_k, topk, p, out_idx,
                             out_score, stats, ws, stream);
  return e == hipSuccess ? SI_OK : SI_ERR_DEVICE;
}
