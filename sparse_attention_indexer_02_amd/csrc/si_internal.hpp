// Internal declarations and device helpers of the sparse-indexer library.
// Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_indexer.h"

namespace si {

constexpr int kWave = 64;

// This thread's wave within the workgroup, as a value the compiler knows to
// be uniform across the wave (so that what is derived from it - row
// indices, buffer resources - stays in scalar registers).
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---------------------------------------------------------------------------
// Orderable 32-bit keys: larger key <=> larger float.  -0 is folded onto +0
// so that IEEE-equal scores tie and fall through to the index.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// 64-bit composite: score key high, complemented index low.  Sorting
// composites descending gives (score desc, index asc); 0 sorts after
// everything real.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(~idx);
}
__device__ __forceinline__ uint32_t comp_key(uint64_t c) { return (uint32_t)(c >> 32); }
__device__ __forceinline__ uint32_t comp_idx(uint64_t c) { return ~(uint32_t)c; }

// Row r sees keys [off, off + vis): vis = clamp(vis_len[r], 0,
// min(max_vis, n_k - off)); a bad offset sees nothing.
__device__ __forceinline__ int64_t visible_len(const int32_t* vis_len, const int64_t* row_off,
                                               int r, int64_t n_k, int64_t max_vis,
                                               int64_t* off_out) {
  int64_t o = row_off ? row_off[r] : 0;
  int64_t v = vis_len[r];
  if (o < 0 || o > n_k) {
    *off_out = 0;
    return 0;
  }
  v = v < 0 ? 0 : v;
  v = v > max_vis ? max_vis : v;
  v = v > n_k - o ? n_k - o : v;
  *off_out = o;
  return v;
}

// ---------------------------------------------------------------------------
// Block-wide helpers (blockDim.x == THREADS, multiple of 64).
// ---------------------------------------------------------------------------
// Wavefront scan and reductions from the ROCm device library (DPP row
// shifts and broadcasts; every lane of the wave must be active).
extern "C" __device__ int __ockl_wfscan_add_i32(int, bool);
extern "C" __device__ unsigned __ockl_wfred_max_u32(unsigned);
extern "C" __device__ unsigned __ockl_wfred_min_u32(unsigned);
extern "C" __device__ unsigned __ockl_wfred_or_u32(unsigned);

__device__ __forceinline__ int wave_incl_scan(int x) { return __ockl_wfscan_add_i32(x, true); }

// Exclusive prefix sum over the block; returns the thread's exclusive
// prefix, *total gets the block total.  `scratch` needs THREADS/64 ints.
template <int THREADS>
__device__ __forceinline__ int block_excl_scan(int x, int* scratch, int* total) {
  constexpr int NW = THREADS / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = wave_incl_scan(x);
  if (lane == 63) scratch[wid] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    int v = scratch[i];
    base += (i < wid) ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

// ---------------------------------------------------------------------------
// Radix select of the K-th largest 32-bit key among n items, digits of
// 11/11/10 bits from the top.  load(i) returns item i's key.  Returns the
// exact key T of the K-th largest item; *n_gt gets the number of items
// strictly greater than T (< K).  Requires 1 <= K <= n.  hist: 2048 ints of
// shared memory; red: THREADS/64 + 4 ints of shared memory.
// ---------------------------------------------------------------------------
template <int THREADS, typename Load>
__device__ uint32_t radix_select_kth(Load load, int64_t n, int64_t K, int* hist, int* red,
                                     int64_t* n_gt) {
  uint32_t prefix = 0, pmask = 0;
  int64_t remaining = K;  // rank of the target among items matching prefix
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const int nb = 1 << widths[pass];
    const uint32_t dmask = (uint32_t)(nb - 1);
    for (int i = threadIdx.x; i < nb; i += THREADS) hist[i] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += THREADS) {
      uint32_t u = load(i);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> sh) & dmask], 1);
    }
    __syncthreads();
    // Each thread owns a contiguous run of bins, counted from the top digit.
    const int per = nb / THREADS > 0 ? nb / THREADS : 1;
    int first = nb - 1 - (int)threadIdx.x * per;  // highest bin of this thread
    int cnt = 0;
    if ((int)threadIdx.x * per < nb)
      for (int j = 0; j < per; ++j) cnt += hist[first - j];
    int tot;
    int above = block_excl_scan<THREADS>(cnt, red, &tot);  // items in higher bins
    if ((int)threadIdx.x * per < nb && above < remaining && above + cnt >= remaining) {
      int acc = above;
      for (int j = 0; j < per; ++j) {
        int h = hist[first - j];
        if (acc + h >= remaining) {
          red[THREADS / 64] = first - j;
          red[THREADS / 64 + 1] = acc;
          break;
        }
        acc += h;
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)red[THREADS / 64];
    remaining -= red[THREADS / 64 + 1];
    prefix |= digit << sh;
    pmask |= dmask << sh;
    __syncthreads();
  }
  *n_gt = K - remaining;
  return prefix;
}

// In-shared-memory bitonic sort of P (power of two) 64-bit items, descending.
template <int THREADS>
__device__ void bitonic_sort_desc(uint64_t* a, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (P >> 1); t += THREADS) {
        int i = 2 * stride * (t / stride) + (t % stride);
        int j = i + stride;
        uint64_t x = a[i], y = a[j];
        bool desc = (i & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          a[i] = y;
          a[j] = x;
        }
      }
      __syncthreads();
    }
  }
}

__host__ __device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ---------------------------------------------------------------------------
// Host-side launchers (each returns hipSuccess or the launch error).
// ---------------------------------------------------------------------------
struct ScoreArgs {
  const void* q;
  si_dtype q_dtype;
  const void* k;
  si_dtype k_dtype;
  const float* k_scale;
  const float* w;
  int64_t w_row_stride;
  const int64_t* k_row_offset;
  const int32_t* vis_len;
  int32_t n_q, H, D;
  int64_t n_k, max_vis;
  float* scores;        // [n_q, score_stride]
  int64_t score_stride;
  // optional (per-row keys only): keep s >= filter_tau[r]; survivor masks
  // per 32-key tile in filter_bitmap [n_q, filter_words], scores stored for
  // survivors only, survivor counts per key chunk and wave in
  // filter_chunk_cnt [n_q, rows_key_chunks(max_vis), 4]
  const float* filter_tau = nullptr;
  uint32_t* filter_bitmap = nullptr;
  int64_t filter_words = 0;
  int32_t* filter_chunk_cnt = nullptr;
};
// Keys per workgroup of the per-row (decode layout) score kernels.
constexpr int64_t kRowsChunk = 4096;
// Row of a workgroup in a (rows x chunks) grid over ragged rows.  Workgroups go
// to the XCDs and their shader engines round robin in launch order, so with
// the row as the fast grid index every engine would take a fixed subset of
// the rows (all of their chunks), and ragged rows would leave engines idle
// while others work through long rows.  Each chunk column rotates the rows by
// its index instead, so a row's chunks spread over the engines.
__device__ __forceinline__ int rows_grid_row() {
  const unsigned n = gridDim.x;
  return (int)((blockIdx.x + n - blockIdx.y % n) % n);
}

inline int64_t rows_key_chunks(int64_t max_vis) { return (max_vis + kRowsChunk - 1) / kRowsChunk; }
hipError_t launch_score(const ScoreArgs& a, hipStream_t st);
bool score_mfma_supported(const ScoreArgs& a);
// Decode top-K with a prior threshold (per-row keys on the MFMA path).
size_t prior_workspace_bytes(int64_t n_q, int64_t max_vis, int K);
hipError_t launch_prior_topk(const ScoreArgs& sa, const int32_t* prior, int prior_width, int K,
                             int32_t* out_idx, float* out_score, float* out_tau,
                             int32_t* out_count, void* ws, hipStream_t st);

struct TopkArgs {
  const float* scores;  // row r at scores + r * stride
  int64_t stride;
  const int32_t* vis_len;  // null: every row has max_vis items
  const int64_t* k_row_offset;
  int64_t n_k, max_vis;
  int32_t n_rows;
  int32_t K;
  int32_t* out_idx;     // [n_rows, K]
  float* out_score;     // [n_rows, K] or null
  const int32_t* id_map = nullptr;     // optional increasing map position -> id
  const int32_t* row_list = nullptr;   // optional: only rows row_list[0 .. *row_count)
  const int32_t* row_count = nullptr;
  int64_t id_map_stride = 0;           // row r maps through id_map + r * id_map_stride
  int32_t chunk = 0;                   // > 0: block y takes positions [y chunk, (y+1) chunk)
  int64_t out_stride = 0;              // output row stride (0: K); chunk y writes at y K
  int32_t len_levels = 0;              // row length = the visible length after this many chunk
                                       // passes (each keeps min(K, chunk) per 8192-chunk)
  // optional segment-witness merge of each final output row (context
  // lengths, S, keep, budget B = min(max_replacements, K - keep))
  const int32_t* wit_lens = nullptr;
  int32_t wit_S = 0, wit_keep = 0, wit_B = 0;
  void* workspace = nullptr;           // candidate lists for rows longer than one block
  size_t workspace_bytes = 0;
};
// Top-K of each row.  Rows of at most 8192 scores with K <= 2048 take one
// workgroup each; longer rows are cut into 8192-score chunks whose top-K
// sets (in id order) are selected from again (needs topk_workspace_bytes of
// workspace; without it, or for K > 2048, a single-workgroup radix select).
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// The one-workgroup block top-K's limits (rows of at most this many scores,
// K at most this).
constexpr int kBlockTopkMaxN = 8192;
constexpr int kBlockTopkMaxK = 2048;
size_t topk_workspace_bytes(int64_t n_rows, int64_t max_vis, int K);
constexpr int kMaxTopk = 4096;
// Score and top-K of the prefill layout in one kernel: the shapes it takes
// (shared bf16 keys in one key segment, rows of at most 8192 keys, K <=
// 2048), and the launch (ta.scores must be a.scores with stride max_vis).
bool score_topk_fused_supported(const ScoreArgs& a, int K);
hipError_t launch_score_topk_fused(const ScoreArgs& a, const TopkArgs& ta, hipStream_t st);
hipError_t launch_score_rows_listed(const ScoreArgs& a, const int32_t* row_list,
                                    const int32_t* row_count, hipStream_t st);

hipError_t launch_block_positions(const int32_t* blocks, int32_t n_q, int32_t heads,
                                  int32_t width, const int64_t* qpos, int64_t n_pos, int32_t bs,
                                  int32_t* out, int32_t out_width, int32_t* count, hipStream_t st);
hipError_t launch_gather_slots(const int32_t* idx, int32_t rows, int32_t width,
                               const int32_t* lens, const int64_t* row_start,
                               const int32_t* table, int32_t ppr, int32_t page, int64_t* out,
                               hipStream_t st);

hipError_t launch_witness(int32_t* idx, int32_t rows, int32_t topk, const int32_t* lens,
                          int32_t S, int32_t keep, int32_t B, hipStream_t st);

}  // namespace si
