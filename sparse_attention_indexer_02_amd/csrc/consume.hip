// The step after selection: what the sparse attention that consumes a
// selection reads.
//
//  * block_positions: the positions a block list covers (ferrox-core
//    block_sparse.rs, the positions helper's doc comment): ascending,
//    deduplicated, and
//    clipped to the keys that exist and to the query's own position.  Lists
//    of at most 64 entries take one wave each (block_positions_wave, below);
//    longer ones one 256-thread workgroup each.  A list's entries
//    become 64-bit keys, larger for lower blocks and 0 for entries that
//    cover nothing (padding, blocks past the query or the keys); a list that
//    is not already in descending key order (block_sparse_select's are) is
//    bitonic-sorted in LDS.  The first of each run of equal keys keeps its
//    block's clipped length, a block scan gives each block's output offset,
//    and thread t writes output slots t + 256 i, each finding its block by a
//    binary search over the offsets (coalesced 1 KB stores per iteration).
//  * gather_slots: the KV slot of every entry of a selection row (Segment
//    Witnesses, Implementation rule and contracts: Coordinates; entries are
//    row-relative, in [0, L_r) when they name a token): flat
//    row_start[r] + x, or paged table[r][x / page] * page + x % page (the
//    block-sparse page's 128-token block is the KV page); -1 otherwise.
#include "si_internal.hpp"

namespace si {

constexpr int kPosThreads = 256;

__global__ __launch_bounds__(kPosThreads) void block_positions(
    const int32_t* __restrict__ blocks, int width, int heads, const int64_t* __restrict__ qpos,
    int64_t n_pos, int bs, int32_t* __restrict__ out, int64_t out_width,
    int32_t* __restrict__ count) {
  extern __shared__ uint64_t key[];  // [P] keys, then [P] int offsets
  __shared__ int red[kPosThreads / 64 + 4];
  const int t = threadIdx.x;
  const int64_t l = blockIdx.x;
  const int P = next_pow2(width > 1 ? width : 1);
  int* off = reinterpret_cast<int*>(key + P);
  const int64_t qp = qpos[l / heads];
  const int64_t lim = qp < 0 ? 0 : (qp + 1 < n_pos ? qp + 1 : n_pos);  // visible positions
  const int64_t nbv = (lim + bs - 1) / bs;                              // blocks that can cover any
  const int32_t* src = blocks + l * width;
  for (int i = t; i < P; i += kPosThreads) {
    const int32_t b = i < width ? src[i] : -1;
    key[i] = (b >= 0 && b < nbv) ? ((1ull << 32) | (uint64_t)(~(uint32_t)b)) : 0ull;
  }
  __syncthreads();
  int unordered = 0;
  for (int i = t; i + 1 < P; i += kPosThreads) unordered |= key[i] < key[i + 1] ? 1 : 0;
  if (__syncthreads_or(unordered)) bitonic_sort_desc<kPosThreads>(key, P);
  // thread t owns entries [t per, (t + 1) per): their clipped lengths
  const int per = P > kPosThreads ? P / kPosThreads : 1;
  const int i0 = t * per;
  auto len_of = [&](int i) -> int {
    if (i >= P) return 0;
    const uint64_t k = key[i];
    if (k == 0ull || (i > 0 && key[i - 1] == k)) return 0;  // nothing, or a repeat
    const int64_t start = (int64_t)(~(uint32_t)k) * bs;
    const int64_t end = start + bs < lim ? start + bs : lim;
    return (int)(end - start);
  };
  int mine = 0;
  for (int j = 0; j < per; ++j) mine += len_of(i0 + j);
  int total;
  int run = block_excl_scan<kPosThreads>(mine, red, &total);
  for (int j = 0; j < per; ++j) {
    if (i0 + j < P) off[i0 + j] = run;
    run += len_of(i0 + j);
  }
  __syncthreads();
  int32_t* o = out + l * out_width;
  for (int64_t s = t; s < out_width; s += kPosThreads) {
    int32_t v = -1;
    if (s < total) {
      // the last entry whose offset is <= s: the block covering slot s
      // (zero-length entries share the offset of the entry after them)
      int lo = 0, hi = P - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= s) lo = mid; else hi = mid - 1;
      }
      v = (int32_t)((int64_t)(~(uint32_t)key[lo]) * bs + (s - off[lo]));
    }
    o[s] = v;
  }
  if (t == 0 && count) count[l] = total;
}

// Lists of at most 64 entries: one wave per list, four per workgroup, no
// barriers.  Lane j holds entry j; an unordered list is bitonic-sorted
// across the lanes; a wave scan gives the offsets; each lane writes four
// consecutive slots per 1 KB wave store (as one 16-byte store when rows are
// 16-byte aligned), finding the first slot's block by a binary search and
// the next three by stepping.
constexpr int kPosWaveLists = 4;

__device__ __forceinline__ uint64_t join_u64(uint32_t lo, uint32_t hi) {
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  return join_u64(__shfl_xor((uint32_t)v, m), __shfl_xor((uint32_t)(v >> 32), m));
}
// lane + 1's value (lane 63: its own)
__device__ __forceinline__ uint64_t shfl_next_u64(uint64_t v) {
  return join_u64(__shfl_down((uint32_t)v, 1), __shfl_down((uint32_t)(v >> 32), 1));
}
// lane - 1's value (lane 0: its own)
__device__ __forceinline__ uint64_t shfl_prev_u64(uint64_t v) {
  return join_u64(__shfl_up((uint32_t)v, 1), __shfl_up((uint32_t)(v >> 32), 1));
}

__global__ __launch_bounds__(64 * kPosWaveLists) void block_positions_wave(
    const int32_t* __restrict__ blocks, int width, int heads, int64_t lists,
    const int64_t* __restrict__ qpos, int64_t n_pos, int bs, int32_t* __restrict__ out,
    int64_t out_width, bool vec4, int32_t* __restrict__ count) {
  __shared__ int offw[kPosWaveLists][64];
  __shared__ int startw[kPosWaveLists][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t l = (int64_t)blockIdx.x * kPosWaveLists + wv;
  if (l >= lists) return;
  const int32_t b = lane < width ? blocks[l * width + lane] : -1;
  const int64_t qp = qpos[l / heads];
  const int64_t lim = qp < 0 ? 0 : (qp + 1 < n_pos ? qp + 1 : n_pos);
  const int64_t nbv = (lim + bs - 1) / bs;
  uint64_t key = (b >= 0 && b < nbv) ? ((1ull << 32) | (uint64_t)(~(uint32_t)b)) : 0ull;
  // descending keys = ascending blocks, entries covering nothing last
  if (__any(lane < 63 && key < shfl_next_u64(key))) {
    for (int size = 2; size <= 64; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const uint64_t other = shfl_xor_u64(key, stride);
        const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
        const uint64_t mx = key > other ? key : other, mn = key > other ? other : key;
        key = (lower == desc) ? mx : mn;
      }
  }
  const uint64_t prev = shfl_prev_u64(key);
  const bool keep = key != 0ull && (lane == 0 || prev != key);
  const int start = (int)((int64_t)(~(uint32_t)key) * bs);  // < lim when kept
  int len = 0;
  if (keep) {
    const int64_t end = (int64_t)start + bs < lim ? (int64_t)start + bs : lim;
    len = (int)(end - start);
  }
  const int incl = wave_incl_scan(len);
  const int total = __shfl(incl, 63);
  offw[wv][lane] = incl - len;
  startw[wv][lane] = start;
  __builtin_amdgcn_wave_barrier();
  const int* off = offw[wv];
  const int* st = startw[wv];
  int32_t* o = out + l * out_width;
  // a list of whole blocks with no repeats (a selection's, but for its
  // clipped last block): slot s lies in kept entry s / bs
  const uint64_t kept = __ballot(keep);
  const int nk = __popcll(kept);
  const bool whole = kept == (nk == 64 ? ~0ull : ((1ull << nk) - 1ull)) &&
                     !__any(keep && lane != nk - 1 && len != bs);
#pragma unroll 4
  for (int64_t base = 4 * lane; base < out_width; base += 256) {
    int32_t v[4];
    if (whole && (bs & 3) == 0) {
      // the four slots share a block
      const uint32_t s = (uint32_t)base;
      const uint32_t q = s / (uint32_t)bs, e = q < 63u ? q : 63u;
      const int32_t v0 = st[e] + (int32_t)(s - e * (uint32_t)bs);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = s + j < (uint32_t)total ? v0 + j : -1;
    } else if (whole) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t s = (uint32_t)(base + j);
        const uint32_t q = s / (uint32_t)bs, e = q < 63u ? q : 63u;
        v[j] = s < (uint32_t)total ? st[e] + (int32_t)(s - e * (uint32_t)bs) : -1;
      }
    }
    int e = 0;
    if (!whole && base < total) {
      int lo = 0, hi = 63;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= base) lo = mid; else hi = mid - 1;
      }
      e = lo;
    }
    if (!whole) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t s = base + j;
        if (s < total) {
          while (e < 63 && off[e + 1] <= s) ++e;
          v[j] = st[e] + (int32_t)(s - off[e]);
        } else {
          v[j] = -1;
        }
      }
    }
    if (vec4) {
      // streamed out: the consumer reads it, this kernel never does
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(i32x4{v[0], v[1], v[2], v[3]},
                                  reinterpret_cast<i32x4*>(o + base));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (base + j < out_width) o[base + j] = v[j];
    }
  }
  if (lane == 0 && count) count[l] = total;
}

hipError_t launch_block_positions(const int32_t* blocks, int32_t n_q, int32_t heads,
                                  int32_t width, const int64_t* qpos, int64_t n_pos, int32_t bs,
                                  int32_t* out, int32_t out_width, int32_t* count,
                                  hipStream_t st) {
  const int64_t lists = (int64_t)n_q * heads;
  if (lists == 0) return hipSuccess;
  if (width <= 64) {
    const bool vec4 = out_width % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    hipLaunchKernelGGL(block_positions_wave,
                       dim3((unsigned)((lists + kPosWaveLists - 1) / kPosWaveLists)),
                       dim3(64 * kPosWaveLists), 0, st, blocks, width, heads, lists, qpos, n_pos,
                       bs, out, (int64_t)out_width, vec4, count);
    return hipGetLastError();
  }
  const int P = next_pow2(width > 1 ? width : 1);
  const size_t lds = (size_t)P * (sizeof(uint64_t) + sizeof(int));
  hipLaunchKernelGGL(block_positions, dim3((unsigned)lists), dim3(kPosThreads), lds, st, blocks,
                     width, heads, qpos, n_pos, bs, out, (int64_t)out_width, count);
  return hipGetLastError();
}

constexpr int kGatherThreads = 256;
constexpr int kGatherPer = 4;  // entries per thread

// Grid (rows, ceil(width / 1024)); thread t of workgroup (r, c) takes
// entries c 1024 + t + 256 j of row r.
__global__ __launch_bounds__(kGatherThreads) void gather_slots_k(
    const int32_t* __restrict__ idx, int width, const int32_t* __restrict__ lens,
    const int64_t* __restrict__ row_start, const int32_t* __restrict__ table, int ppr, int page,
    int64_t* __restrict__ out) {
  const int64_t r = blockIdx.x;
  const int base = (int)blockIdx.y * (kGatherThreads * kGatherPer) + (int)threadIdx.x;
  const int32_t L = lens[r];
  const int64_t rs = row_start ? row_start[r] : 0;
  const int32_t* tr = table ? table + r * ppr : nullptr;
  int32_t x[kGatherPer];
#pragma unroll
  for (int j = 0; j < kGatherPer; ++j) {
    const int i = base + j * kGatherThreads;
    x[j] = i < width ? idx[r * width + i] : -1;
  }
#pragma unroll
  for (int j = 0; j < kGatherPer; ++j) {
    const int i = base + j * kGatherThreads;
    if (i >= width) continue;
    int64_t slot = -1;
    if (x[j] >= 0 && x[j] < L) {
      if (!tr) {
        slot = rs + x[j];
      } else {
        const uint32_t ux = (uint32_t)x[j], up = (uint32_t)page;
        const uint32_t pg = ux / up;
        if (pg < (uint32_t)ppr) {
          const int32_t id = tr[pg];
          if (id >= 0) slot = (int64_t)id * page + (int64_t)(ux - pg * up);
        }
      }
    }
    out[r * width + i] = slot;
  }
}

hipError_t launch_gather_slots(const int32_t* idx, int32_t rows, int32_t width,
                               const int32_t* lens, const int64_t* row_start,
                               const int32_t* table, int32_t ppr, int32_t page, int64_t* out,
                               hipStream_t st) {
  if (rows == 0 || width == 0) return hipSuccess;
  const int64_t chunks = ((int64_t)width + kGatherThreads * kGatherPer - 1) /
                         (kGatherThreads * kGatherPer);
  hipLaunchKernelGGL(gather_slots_k, dim3((unsigned)rows, (unsigned)chunks), dim3(kGatherThreads),
                     0, st, idx, width, lens, row_start, table, ppr, page, out);
  return hipGetLastError();
}

}  // namespace si
