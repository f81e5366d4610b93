// Per-row top-K under the total order (score desc, index asc), -0 == +0
// (DoSA reading notes, section 1: one consistent total order makes tied ids
// reproducible; the final selection is by full score).
//
// Kernels:
//  * topk_block: rows of at most 8192 scores, K <= 2048, one 512-thread
//    workgroup per row holding the row in registers (steps in
//    topk_block.hpp).  Longer rows (K <= 2048, with a workspace) are cut
//    into 8192-score chunks whose top-K sets (in ascending position, so in
//    id order), with the chunks' position maps, are selected from again by
//    the same kernel until one chunk remains, which is ordered (each level's row lengths follow from the original ones,
//    TopkArgs::len_levels).
//  * topk_rows: K > 2048, or a long row without a workspace.  One
//    512-thread workgroup per row; rows up to 8192 scores are staged in LDS,
//    longer ones re-read per pass; a 3-pass radix select (11/11/10-bit
//    digits) finds the K-th key, ties at it are taken in index order, and a
//    bitonic sort of (key, ~index) composites orders them.
#include "topk_block.hpp"

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
  // a NaN score ranks (and is reported) as -inf, as in the block kernel;
  // order_key folds -0 onto +0
  auto key_at = [&](int64_t i) -> uint32_t {
    const float v = row[i];
    return order_key(v == v ? v : -__builtin_inff());
  };
  if (staged)
    for (int64_t i = threadIdx.x; i < n; i += T) keys[i] = key_at(i);
  if (threadIdx.x == 0) counter = 0;
  __syncthreads();
  auto load = [&](int64_t i) -> uint32_t { return staged ? keys[i] : key_at(i); };

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
      oi[t] = a.id_map ? a.id_map[(int64_t)r * a.id_map_stride + idx] : (int32_t)idx;
      if (os) os[t] = key_to_float(comp_key(c));
    } else {
      oi[t] = -1;
      if (os) os[t] = -__builtin_inff();
    }
  }
}

// eight waves per SIMD (64 VGPRs): four rows' 32 waves fill a CU
template <bool WIT, bool CHUNK>
__global__ __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(8))) void topk_block(
    TopkArgs a) {
  __shared__ TopkSmem<kBT> S;
  // (a chunk pass's grid is rows x chunks: rotated as for the decode score)
  int r = rows_grid_row();
  if (a.row_list) {
    if (r >= *a.row_count) return;
    r = a.row_list[r];
  } else {
    r = a.n_rows - 1 - r;  // causal rows grow with the index: longest first
  }
  topk_row_block<kBT, kBN / kBT, WIT, CHUNK>(a, r, (int)blockIdx.y, S);
}

// Bytes of one chunk level (candidate ids + scores + per-row counts), and
// the number of chunks per row of a level with rows of at most len scores.
static int64_t chunks_of(int64_t len) { return (len + kBN - 1) / kBN; }
static size_t level_bytes(int64_t n_rows, int64_t len, int K) {
  const size_t cand = (size_t)n_rows * (size_t)chunks_of(len) * (size_t)K;
  return (cand * 8 + 255) & ~(size_t)255;
}

size_t topk_workspace_bytes(int64_t n_rows, int64_t max_vis, int K) {
  if (K > kBK || max_vis <= kBN || n_rows <= 0) return 0;
  size_t total = 0;
  for (int64_t len = max_vis; len > kBN; len = chunks_of(len) * K) total += level_bytes(n_rows, len, K);
  return total;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_rows);
  if (a.K <= kBK && a.max_vis <= kBN) {
    if (a.wit_lens) hipLaunchKernelGGL((topk_block<true, false>), grid, dim3(kBT), 0, st, a);
    else hipLaunchKernelGGL((topk_block<false, false>), grid, dim3(kBT), 0, st, a);
    return hipGetLastError();
  }
  const size_t need = topk_workspace_bytes(a.n_rows, a.max_vis, a.K);
  if (a.K > kBK || a.workspace == nullptr || a.workspace_bytes < need) {
    hipLaunchKernelGGL(topk_rows, grid, dim3(kTopkThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    // this kernel has no fused witness merge: the merge kernel follows
    // (row lists do not occur with a witness merge)
    if (e == hipSuccess && a.wit_lens)
      e = launch_witness(a.out_idx, a.n_rows, a.K, a.wit_lens, a.wit_S, a.wit_keep, a.wit_B, st);
    return e;
  }
  // chunk passes until a row's candidates fit one block, then the last pass
  TopkArgs cur = a;
  cur.chunk = 0;
  cur.out_stride = 0;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  int64_t len = a.max_vis;
  while (len > kBN) {
    const int64_t nch = chunks_of(len);
    const int64_t cstride = nch * a.K;
    int32_t* cidx = reinterpret_cast<int32_t*>(ws);
    float* csc = reinterpret_cast<float*>(ws + (size_t)a.n_rows * cstride * 4);
    TopkArgs L = cur;
    L.chunk = kBN;
    L.out_idx = cidx;
    L.out_score = csc;
    L.out_stride = cstride;
    hipLaunchKernelGGL((topk_block<false, true>), dim3((unsigned)a.n_rows, (unsigned)nch), dim3(kBT),
                       0, st, L);
    // the next level's rows: the candidates this pass keeps, at the same
    // positions as the level's rows (lengths follow from the original ones)
    cur.scores = csc;
    cur.stride = cstride;
    cur.len_levels += 1;
    cur.id_map = cidx;
    cur.id_map_stride = cstride;
    ws += level_bytes(a.n_rows, len, a.K);
    len = cstride;
  }
  cur.out_idx = a.out_idx;
  cur.out_score = a.out_score;
  if (a.wit_lens) hipLaunchKernelGGL((topk_block<true, false>), grid, dim3(kBT), 0, st, cur);
  else hipLaunchKernelGGL((topk_block<false, false>), grid, dim3(kBT), 0, st, cur);
  return hipGetLastError();
}

}  // namespace si
