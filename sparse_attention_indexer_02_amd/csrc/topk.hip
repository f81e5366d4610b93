// Per-row top-K under the total order (score desc, index asc), -0 == +0
// (DoSA reading notes, section 1: one consistent total order makes tied ids
// reproducible; the final selection is by full score).
//
// One workgroup per row.  Rows up to kStage scores are staged in LDS as
// orderable keys (one HBM read); longer rows are re-read per pass.  A 3-pass
// radix select (11/11/10-bit digits, LDS histograms) finds the exact key T
// of the K-th item; items above T are gathered with an LDS counter and the
// ties at T are taken in index order with a block scan; a bitonic sort of
// (key, ~index) composites orders the K winners.
#include "si_internal.hpp"

namespace si {

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

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows, dim3((unsigned)a.n_rows), dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace si
