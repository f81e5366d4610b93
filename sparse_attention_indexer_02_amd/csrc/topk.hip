// Per-row top-K under the total order (score desc, index asc), -0 == +0
// (DoSA reading notes, section 1: one consistent total order makes tied ids
// reproducible; the final selection is by full score).
//
// Two kernels:
//  * topk_wave<PER>: rows of at most 64*PER scores (<= 8192), K <= 2048.
//    One wavefront per row and no cross-wave synchronisation: the row
//    lives in registers, every row-wide step is one pass over them, and
//    ordered compaction is a ballot prefix.  See the kernel for the steps.
//  * topk_rows: any length and K <= 4096 (long decode rows, DoSA's seed and
//    fallback rows).  One 512-thread workgroup per row; rows up to 8192
//    scores are staged in LDS, longer ones re-read per pass; a 3-pass radix
//    select (11/11/10-bit digits) finds the K-th key, ties at it are taken in
//    index order, and a bitonic sort of (key, ~index) composites orders them.
#include "si_internal.hpp"

namespace si {

// ---------------------------------------------------------------------------
// Generic kernel.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 512;
constexpr int kStage = 8192;

__global__ __launch_bounds__(kTopkThreads) void topk_rows(TopkArgs a) {
  constexpr int T = kTopkThreads;
  __shared__ uint32_t keys[kStage];
  __shared__ int hist[2048];
  __shared__ uint64_t sortbuf[kMaxTopk];
  __shared__ int red[T / 64 + 4];
  __shared__ int counter;

  int r = blockIdx.x;
  if (a.row_list) {
    if (r >= *a.row_count) return;
    r = a.row_list[r];
  }
  int64_t off;
  const int64_t n =
      a.vis_len ? visible_len(a.vis_len, a.k_row_offset, r, a.n_k, a.max_vis, &off) : a.max_vis;
  const float* row = a.scores + (int64_t)r * a.stride;
  const int K = a.K;
  const bool staged = n <= kStage;
  if (staged)
    for (int64_t i = threadIdx.x; i < n; i += T) keys[i] = order_key(row[i]);
  if (threadIdx.x == 0) counter = 0;
  __syncthreads();
  auto load = [&](int64_t i) -> uint32_t { return staged ? keys[i] : order_key(row[i]); };

  const int cnt = (int)(n < K ? n : K);
  const int P = next_pow2(cnt > 1 ? cnt : 1);
  if (n <= K) {
    for (int64_t i = threadIdx.x; i < n; i += T) sortbuf[i] = composite(load(i), (uint32_t)i);
  } else {
    int64_t n_gt;
    const uint32_t thr = radix_select_kth<T>(load, n, K, hist, red, &n_gt);
    // strictly greater: any slot order
    for (int64_t i = threadIdx.x; i < n; i += T) {
      uint32_t u = load(i);
      if (u > thr) sortbuf[atomicAdd(&counter, 1)] = composite(u, (uint32_t)i);
    }
    // ties at the threshold: the lowest indices first
    const int need = K - (int)n_gt;
    int taken = 0;
    for (int64_t base = 0; base < n && taken < need; base += T) {
      int64_t i = base + threadIdx.x;
      int flag = (i < n && load(i) == thr) ? 1 : 0;
      int tot;
      int rank = block_excl_scan<T>(flag, red, &tot);
      if (flag && taken + rank < need) sortbuf[n_gt + taken + rank] = composite(thr, (uint32_t)i);
      taken += tot;
    }
  }
  for (int i = cnt + threadIdx.x; i < P; i += T) sortbuf[i] = 0ull;
  __syncthreads();
  bitonic_sort_desc<T>(sortbuf, P);
  int32_t* oi = a.out_idx + (int64_t)r * K;
  float* os = a.out_score ? a.out_score + (int64_t)r * K : nullptr;
  for (int t = threadIdx.x; t < K; t += T) {
    if (t < cnt) {
      uint64_t c = sortbuf[t];
      uint32_t idx = comp_idx(c);
      oi[t] = a.id_map ? a.id_map[idx] : (int32_t)idx;
      if (os) os[t] = key_to_float(comp_key(c));
    } else {
      oi[t] = -1;
      if (os) os[t] = -__builtin_inff();
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of at most 8192 scores, K <= 2048: one 256-thread workgroup per row,
// thread t owning positions [32 t, 32 t + 32) in registers (16-byte loads),
// so index order is thread order and every ordered step is one block scan.
//  A. load, make orderable keys, histogram their top 11 bits (coarse bins,
//     4 replicas of 16-bit counters against atomic contention), row range;
//  B. scan of the coarse bins from the top: bin b1 holds the K-th item; the
//     coarse counts become packed (offset << 16 | selected count) per bin;
//  C. list bin b1's keys and refine on the list with the next 11 and 10
//     bits: the exact K-th key T, the count above it and the ties at it (a
//     crowded b1 refines over the registers instead);
//  D. index-ordered compaction: keys > T, then the lowest-index keys == T;
//  E. bucket rank: each coarse bin owns as many buckets as it has selected
//     items, spread linearly over its low 21 key bits (~1 item per bucket
//     for any smooth score density); an item's output slot is its bucket's
//     offset plus the number of same-bucket items ahead of it under
//     (score desc, index asc).
// ---------------------------------------------------------------------------
constexpr int kBT = 256;             // threads per row
constexpr int kBPer = 32;            // positions per thread
constexpr int kBN = kBT * kBPer;     // 8192
constexpr int kBK = 2048;            // largest K
constexpr int kBItems = kBK / kBT;   // 8 dense items per thread

struct BlockSmem {
  // coarse histogram: 4 replicas x 2048 16-bit counters; afterwards words
  // [0, 2048) hold the packed per-bin (offset << 16 | count) and words
  // [2048, 4096) the bucket counters/offsets
  uint32_t coarse[4096];
  // candidate list + refine histogram, then the dense list, then buckets
  union {
    struct {
      uint32_t list[2048];
      uint32_t rh[2048];
    } r;
    uint64_t dense[kBK];
  } x;
};

__device__ __forceinline__ uint32_t coarse_count(const uint32_t* c, int b) {
  uint32_t s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) s += (c[q * 1024 + (b >> 1)] >> ((b & 1) * 16)) & 0xFFFFu;
  return s;
}

// Owner search over nb bins (per thread `per` consecutive bins from the
// top): returns the bin holding the rank-th item, the items above it and
// its own count.  `cnt` is read through `get(b)`.
template <class Get>
__device__ __forceinline__ void block_find_bin(Get get, int nb, int rank, int* red,
                                               uint32_t* bin, int* above, int* count) {
  const int t = threadIdx.x;
  const int per = nb / kBT;
  const int first = nb - 1 - t * per;
  int c = 0;
  for (int j = 0; j < per; ++j) c += (int)get(first - ((j + t) & (per - 1)));
  int tot;
  const int ab = block_excl_scan<kBT>(c, red, &tot);
  if (ab < rank && ab + c >= rank) {
    int acc = ab;
    for (int j = 0; j < per; ++j) {
      const int h = (int)get(first - j);
      if (acc + h >= rank) {
        red[kBT / 64] = first - j;
        red[kBT / 64 + 1] = acc;
        red[kBT / 64 + 2] = h;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
  *bin = (uint32_t)red[kBT / 64];
  *above = red[kBT / 64 + 1];
  *count = red[kBT / 64 + 2];
  __syncthreads();
}

__global__ __launch_bounds__(kBT) void topk_block(TopkArgs a) {
  __shared__ BlockSmem sm;
  __shared__ int red[kBT / 64 + 4];
  __shared__ uint32_t wred[2][kBT / 64];
  __shared__ int lcount;
  const int t = threadIdx.x;
  int r = blockIdx.x;
  if (a.row_list) {
    if (r >= *a.row_count) return;
    r = a.row_list[r];
  }
  int64_t off;
  const int64_t n64 =
      a.vis_len ? visible_len(a.vis_len, a.k_row_offset, r, a.n_k, a.max_vis, &off) : a.max_vis;
  const int n = (int)(n64 < kBN ? n64 : kBN);
  const int K = a.K;
  const int cnt = n < K ? n : K;
  const float* row = a.scores + (int64_t)r * a.stride;
  int32_t* oi = a.out_idx + (int64_t)r * K;
  float* os = a.out_score ? a.out_score + (int64_t)r * K : nullptr;
  const int p0 = kBPer * t;
  if (n <= 0) {
    for (int q = t; q < K; q += kBT) {
      oi[q] = -1;
      if (os) os[q] = -__builtin_inff();
    }
    return;
  }

  // A. load + keys + coarse histogram + key range
  for (int i = t; i < 4096; i += kBT) sm.coarse[i] = 0u;
  if (t == 0) lcount = 0;
  uint32_t u[kBPer];
  {
    const uint32_t* rowb = reinterpret_cast<const uint32_t*>(row);
    const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
#pragma unroll
    for (int v = 0; v < kBPer / 4; ++v) {  // every load in flight before the first use
      const int p = p0 + 4 * v;
      if (vec && p + 4 <= n) {
        const uint4 x = *reinterpret_cast<const uint4*>(rowb + p);
        u[4 * v + 0] = x.x;
        u[4 * v + 1] = x.y;
        u[4 * v + 2] = x.z;
        u[4 * v + 3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[4 * v + e] = p + e < n ? rowb[p + e] : 0u;
      }
    }
  }
  __syncthreads();
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  {
    uint32_t* rep = sm.coarse + (t & 3) * 1024;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const bool valid = p0 + i < n;
      u[i] = valid ? order_key(__uint_as_float(u[i])) : 0u;
      if (valid) {
        kmax = u[i] > kmax ? u[i] : kmax;
        kmin = u[i] < kmin ? u[i] : kmin;
        const uint32_t b = u[i] >> 21;
        atomicAdd(&rep[b >> 1], 1u << ((b & 1u) * 16));
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)kmax, o, 64);
    const uint32_t z = (uint32_t)__shfl_xor((int)kmin, o, 64);
    kmax = y > kmax ? y : kmax;
    kmin = z < kmin ? z : kmin;
  }
  if ((t & 63) == 0) {
    wred[0][t >> 6] = kmax;
    wred[1][t >> 6] = kmin;
  }
  __syncthreads();
  for (int i = 0; i < kBT / 64; ++i) {
    kmax = wred[0][i] > kmax ? wred[0][i] : kmax;
    kmin = wred[1][i] < kmin ? wred[1][i] : kmin;
  }
  const bool select = n > K;

  // B. the coarse bin of the K-th item (or, selecting everything, of the
  //    smallest key), then packed per-bin (offset << 16 | selected count)
  uint32_t b1;
  int ab1, in_bin;
  {
    const int want = select ? K : n;
    block_find_bin([&](int b) { return coarse_count(sm.coarse, b); }, 2048, want, red, &b1, &ab1,
                   &in_bin);
  }
  const int rank = (select ? K : n) - ab1;  // items wanted from bin b1
  {
    // thread t owns bins 2047 - 8 t .. 2040 - 8 t
    uint32_t c8[8];
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b = 2047 - 8 * t - j;
      c8[j] = (uint32_t)b >= b1 ? coarse_count(sm.coarse, b) : 0u;
      if ((uint32_t)b == b1) c8[j] = (uint32_t)rank;
      s += (int)c8[j];
    }
    int tot;
    int o = block_excl_scan<kBT>(s, red, &tot);  // its trailing sync orders the reads
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b = 2047 - 8 * t - j;
      sm.coarse[b] = ((uint32_t)o << 16) | c8[j];
      o += (int)c8[j];
    }
  }
  __syncthreads();

  // C. exact threshold key inside bin b1
  uint32_t thr = 0u;
  int n_gt = 0, n_eq = 0;
  if (select) {
    uint32_t d2, d3;
    int ab2, ab3, c2;
    for (int i = t; i < 2048; i += kBT) sm.x.r.rh[i] = 0u;
    if (in_bin <= 2048) {
#pragma unroll
      for (int i = 0; i < kBPer; ++i)
        if (p0 + i < n && (u[i] >> 21) == b1) sm.x.r.list[atomicAdd(&lcount, 1)] = u[i];
      __syncthreads();
      for (int i = t; i < in_bin; i += kBT) {
        const uint32_t v = sm.x.r.list[i];
        atomicAdd(&sm.x.r.rh[(v >> 10) & 2047u], 1u);
      }
    } else {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kBPer; ++i)
        if (p0 + i < n && (u[i] >> 21) == b1) atomicAdd(&sm.x.r.rh[(u[i] >> 10) & 2047u], 1u);
    }
    __syncthreads();
    block_find_bin([&](int b) { return sm.x.r.rh[b]; }, 2048, rank, red, &d2, &ab2, &c2);
    const uint32_t pre2 = (b1 << 21) | (d2 << 10);
    for (int i = t; i < 1024; i += kBT) sm.x.r.rh[i] = 0u;
    __syncthreads();
    if (in_bin <= 2048) {
      for (int i = t; i < in_bin; i += kBT) {
        const uint32_t v = sm.x.r.list[i];
        if ((v >> 10) == (pre2 >> 10)) atomicAdd(&sm.x.r.rh[v & 1023u], 1u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBPer; ++i)
        if (p0 + i < n && (u[i] >> 10) == (pre2 >> 10)) atomicAdd(&sm.x.r.rh[u[i] & 1023u], 1u);
    }
    __syncthreads();
    block_find_bin([&](int b) { return sm.x.r.rh[b]; }, 1024, rank - ab2, red, &d3, &ab3, &n_eq);
    thr = pre2 | d3;
    n_gt = ab1 + ab2 + ab3;
  }

  // D. index-ordered compaction into the dense list
  const int need_eq = select ? K - n_gt : 0;
  {
    int c_gt = 0, c_eq = 0;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const bool valid = p0 + i < n;
      c_gt += (valid && u[i] > thr) ? 1 : 0;
      c_eq += (valid && select && u[i] == thr) ? 1 : 0;
    }
    int tot;
    int eq_before = 0;
    if (need_eq < n_eq) eq_before = block_excl_scan<kBT>(c_eq, red, &tot);  // uniform branch
    int take = need_eq - eq_before;
    take = take < 0 ? 0 : (take > c_eq ? c_eq : take);
    int w = block_excl_scan<kBT>(c_gt + take, red, &tot);
    int taken = 0;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const bool valid = p0 + i < n;
      const bool sel =
          valid && (u[i] > thr || (select && u[i] == thr && taken++ < take));
      if (sel) sm.x.dense[w++] = ((uint64_t)u[i] << 32) | (uint32_t)(~(uint32_t)(p0 + i));
    }
  }
  __syncthreads();

  // E. bucket rank
  uint64_t it[kBItems];
#pragma unroll
  for (int i = 0; i < kBItems; ++i) {
    const int q = kBItems * t + i;
    it[i] = q < cnt ? sm.x.dense[q] : 0ull;
  }
  auto emit = [&](uint32_t dst, uint64_t c) {
    const uint32_t p = ~(uint32_t)c;
    oi[dst] = a.id_map ? a.id_map[p] : (int32_t)p;
    if (os) os[dst] = key_to_float((uint32_t)(c >> 32));
  };
  const uint32_t kmin_sel = select ? thr : kmin;
  if (cnt > 0 && kmin_sel == kmax) {
    // one distinct key: index order, already the dense order
#pragma unroll
    for (int i = 0; i < kBItems; ++i)
      if (kBItems * t + i < cnt) emit((uint32_t)(kBItems * t + i), it[i]);
  } else if (cnt > 0) {
    uint32_t* bcnt = sm.coarse + 2048;  // bucket b at (b & 7) * 256 + (b >> 3)
    auto bsw = [](uint32_t b) { return ((b & 7u) << 8) | (b >> 3); };
    const uint32_t lo_thr = kmin_sel & 0x1FFFFFu;
    uint32_t bk[kBItems];
#pragma unroll
    for (int i = 0; i < kBItems; ++i) {
      bk[i] = 0;
      if (kBItems * t + i < cnt) {
        const uint32_t key = (uint32_t)(it[i] >> 32);
        const uint32_t cb = key >> 21, pk = sm.coarse[cb];
        const uint32_t o = pk >> 16, c = pk & 0xFFFFu;
        const uint32_t lo = cb == b1 ? lo_thr : 0u;
        int sub = (int)((float)((key & 0x1FFFFFu) - lo) * ((float)c / (float)(0x200000u - lo)));
        sub = sub < (int)c - 1 ? sub : (int)c - 1;
        bk[i] = o + (c - 1 - (uint32_t)sub);  // highest keys first
      }
    }
    for (int i = t; i < 2048; i += kBT) bcnt[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kBItems; ++i)
      if (kBItems * t + i < cnt) atomicAdd(&bcnt[bsw(bk[i])], 1u);
    __syncthreads();
    {
      uint32_t c8[8];
      int s = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        c8[j] = bcnt[(j << 8) | t];
        s += (int)c8[j];
      }
      int tot;
      uint32_t o = (uint32_t)block_excl_scan<kBT>(s, red, &tot);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bcnt[(j << 8) | t] = o << 16;  // offset, cursor 0
        o += c8[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kBItems; ++i)
      if (kBItems * t + i < cnt) {
        const uint32_t w = atomicAdd(&bcnt[bsw(bk[i])], 1u);
        sm.x.dense[(w >> 16) + (w & 0xFFFFu)] = it[i];
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kBItems; ++i) {
      if (kBItems * t + i < cnt) {
        const uint32_t w = bcnt[bsw(bk[i])];
        const uint32_t s0 = w >> 16, s1 = s0 + (w & 0xFFFFu);
        uint32_t rk = 0;
        for (uint32_t x = s0; x < s1; ++x) rk += sm.x.dense[x] > it[i] ? 1u : 0u;
        emit(s0 + rk, it[i]);
      }
    }
  }
  for (int q = cnt + t; q < K; q += kBT) {
    oi[q] = -1;
    if (os) os[q] = -__builtin_inff();
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_rows);
  if (a.K <= kBK && a.max_vis <= kBN)
    hipLaunchKernelGGL(topk_block, grid, dim3(kBT), 0, st, a);
  else
    hipLaunchKernelGGL(topk_rows, grid, dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace si
