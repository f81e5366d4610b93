// Per-row top-K with one workgroup and the row in registers, for rows of at
// most 8192 scores and K <= 2048 (the block kernel of the top-K stage and its
// chunk passes, and the top-K phase of the fused prefill kernel).
#pragma once

#include "witness_seg.hpp"

namespace si {

// ---------------------------------------------------------------------------
// Rows of at most 8192 scores, K <= 2048: one workgroup of T threads per
// row, P = 8192 / T scores per thread (the top-K kernel: T = 512, P = 16,
// eight waves per row: with four rows per CU, limited by LDS, the CU holds
// its full 32 waves, and more waves per row measured faster than more
// registers per thread; the fused prefill kernel: T = 256, P = 32).  Thread
// t holds the float4 groups t, t + T, t + 2T, ... of the row (positions
// 4 t + 4 T j + c), so the workgroup's loads of group row j read 16 T bytes
// contiguous, and a row of n scores keeps every wave busy on its first
// ceil(n / 4T) group rows (the rest are skipped uniformly).
//  A. load (a NaN score is taken as -inf) and the row's value range;
//  B. histogram over 4096 bins linear in score value over [vmin, vmax];
//  C. scan from the top bin: the bin b1 holding the K-th item, and per bin
//     the packed (output offset << 16 | selected count);
//  D. the exact K-th value T inside b1: every b1 item counts the b1 items
//     above it when b1 is small, else a radix select on the key bits of
//     b1's items picks T;
//  E. the selected items (> T, then the lowest-index ones == T, found with
//     a position bitmap when T is tied) are scattered grouped by bin; an
//     item's output slot is its bin's offset plus the number of same-bin
//     items ahead of it under (score desc, index asc), counted over the bin
//     four entries at a time (entries past the bin belong to lower bins or
//     are zero, so they never count), and the item is written straight to
//     that slot of the output row.  If some bin holds more than kCrowd
//     selected items (heavy ties, very uneven scores) the row is ordered by
//     a bitonic sort in LDS and written from there.
// A chunk pass (CHUNK) needs the set, not its order: after the selection it
// writes the selected items in ascending position and stops (C skips the
// per-bin offsets; a chunk with at most K items skips B to D).  The final
// pass of a fused witness merge (WIT) also ORs each written id's segment
// bit into the row's occupancy and, once the row is out, writes the
// witnesses of the empty segments.
// Staged items are 64-bit composites: order key << 32 | bin << 13 |
// (8191 - position); composites compare as (score desc, index asc), and the
// bin rides along so the rank step need not recompute it.
// ---------------------------------------------------------------------------
constexpr int kBT = 512;              // threads per row of the top-K kernel
constexpr int kBN = kBlockTopkMaxN;   // row capacity (8192): threads x positions per thread
constexpr int kBK = kBlockTopkMaxK;   // largest K (2048)
constexpr int kBins = 4096;           // value bins
constexpr int kBrute = 256;           // largest b1 ranked item by item
constexpr int kCrowd = 64;            // largest per-bin count ranked by scanning the bin
constexpr int kPosBits = 13;          // positions < kBN
constexpr uint32_t kPosMask = (1u << kPosBits) - 1u;
constexpr int kRowBufWord3 = 0x00020000;  // buffer resource word 3: raw 32-bit dword access

struct alignas(16) BlockSmem {
  uint32_t bins[kBins + 64];  // histogram, then packed (cursor << 16 | selected count);
                              // then one scratch word per lane
  union {
    uint64_t comp[kBK + 4];  // selected composites grouped by bin (+ 4 zero
                             // entries past the last); sorted in place when
                             // a bin is too crowded to rank
    uint32_t sub[2048];      // refine histogram
    uint32_t list[kBrute];   // b1's values
    struct {
      uint32_t bits[kBN / 32];  // positions holding T
      uint32_t pre[kBN / 32];   // exclusive prefix of their popcounts
    } eq;
  } x;
};

// Owner search over nb bins from the top (thread t owns nb/kBT consecutive
// bins, highest first): the bin holding the want-th item from the top, the
// items above it and its count.  get(b) reads bin b's count.
template <int kBT, class Get>
__device__ __forceinline__ void find_from_top(Get get, int nb, int want, int* red, int* bin,
                                              int* above, int* count) {
  const int t = threadIdx.x;
  const int per = nb / kBT;
  const int first = nb - 1 - t * per;
  int c = 0;
  for (int j = 0; j < per; ++j) c += (int)get(first - j);
  int tot;
  const int ab = block_excl_scan<kBT>(c, red, &tot);
  if (ab < want && ab + c >= want) {
    int acc = ab;
    for (int j = 0; j < per; ++j) {
      const int h = (int)get(first - j);
      if (acc + h >= want) {
        red[kBT / 64] = first - j;
        red[kBT / 64 + 1] = acc;
        red[kBT / 64 + 2] = h;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
  *bin = red[kBT / 64];
  *above = red[kBT / 64 + 1];
  *count = red[kBT / 64 + 2];
  __syncthreads();
}

template <int kBT>
struct TopkSmem {
  BlockSmem sm;
  int red[kBT / 64 + 8];
  float fred[2][kBT / 64];
  uint32_t crowd;  // largest selected count of a bin
  uint32_t occ[2];  // fused witness merge: the row's segment occupancy
  int lcount;
};

// One row (or one chunk of a row) with the kBT threads of the calling
// workgroup; every thread must call it (it synchronises the workgroup).
// WIT: the build with the fused witness merge (its extra state costs the
// plain build's register budget, so the plain build leaves it out).
// CHUNK: the build for chunk passes (a.chunk > 0), which end after the
// selection; the final pass (a.chunk == 0) takes CHUNK false.
template <int kBT, int kBPer, bool WIT, bool CHUNK>
__device__ __forceinline__ void topk_row_block(const TopkArgs& a, int r, int cy,
                                               TopkSmem<kBT>& S) {
  static_assert(kBT * kBPer == kBN, "threads x positions per thread = row capacity");
  static_assert(kBPer % 4 == 0 && kBPer <= 32, "float4 groups; one mask bit per position");
  static_assert(kBT >= kBN / 32 && kBT % 64 == 0, "one thread per word of the tie bitmap");
  constexpr int kBGroups = kBPer / 4;   // float4 groups per thread
  constexpr int kBStep = 4 * kBT;       // positions per group row
  constexpr int kBinsPer = kBins / kBT;
  BlockSmem& sm = S.sm;
  int* red = S.red;
  float (*fred)[kBT / 64] = S.fred;
  int& lcount = S.lcount;
  const int t = (int)threadIdx.x;
  const int lane = t & 63, wid = t >> 6;
  int64_t off;
  int64_t n64 =
      a.vis_len ? visible_len(a.vis_len, a.k_row_offset, r, a.n_k, a.max_vis, &off) : a.max_vis;
  // a chunk pass keeps min(K, chunk length) candidates of each 8192-chunk
  for (int l = 0; l < a.len_levels; ++l) {
    const int64_t full = n64 > 0 ? (n64 - 1) / kBN : 0;  // chunks before the last one
    const int64_t last = n64 - full * kBN;
    n64 = n64 > 0 ? full * a.K + (last < a.K ? last : a.K) : 0;
  }
  const int K = a.K;
  // chunk mode: this block takes positions [start, start + chunk) of the row
  // and writes its top-K set, in ascending position, at y K of the output
  // row; an empty chunk
  // writes nothing (the next level never reads it)
  const int64_t start = a.chunk > 0 ? (int64_t)cy * a.chunk : 0;
  if (a.chunk > 0) {
    n64 -= start;
    if (n64 <= 0) return;
    n64 = n64 < a.chunk ? n64 : a.chunk;
  }
  const int n = (int)(n64 < kBN ? n64 : kBN);
  const int cnt = n < K ? n : K;
  const float* row = a.scores + (int64_t)r * a.stride + start;
  const int64_t ostride = a.out_stride > 0 ? a.out_stride : K;
  const int64_t obase = (int64_t)r * ostride + (a.chunk > 0 ? (int64_t)cy * K : 0);
  int32_t* oi = a.out_idx + obase;
  float* os = a.out_score ? a.out_score + obase : nullptr;
  const int32_t* idmap = a.id_map ? a.id_map + (int64_t)r * a.id_map_stride + start : nullptr;
  // fused witness merge of a final row: the segment bits of the ids
  // written, OR-reduced once the row is out
  const bool wit = WIT && a.wit_lens != nullptr && a.chunk == 0;
  const int32_t wL = wit ? a.wit_lens[r] : 0;
  const uint32_t wS = (uint32_t)a.wit_S;
  const uint32_t wSe = wL > 0 ? (wS < (uint32_t)wL ? wS : (uint32_t)wL) : 0u;
  const float wrcp = wL > 0 ? 1.0f / (float)wL : 0.0f;
  if (n <= 0) {
    for (int q = t; q < K; q += kBT) {
      oi[q] = -1;
      if (os) os[q] = -__builtin_inff();
    }
    if (wit && wL > 0) {  // an empty row: every segment takes its witness
      __syncthreads();
      if (wid == 0) write_witnesses(oi, 0ull, (uint32_t)wL, wSe, a.wit_keep, a.wit_B);
    }
    return;
  }
  const bool select = n > K;
  // group rows [0, gfull) are visible everywhere, group row gfull (if
  // < gused) partly; the rest hold nothing.  Bit 4 j + c of vm: position
  // base + kBStep j + c is visible.
  const int base = 4 * t;
  const int gfull = n / kBStep;
  const int gused = (n + kBStep - 1) / kBStep;
  auto pos_of = [&](int i) { return base + kBStep * (i >> 2) + (i & 3); };
  uint32_t vm = gfull >= kBGroups ? 0xFFFFFFFFu : ((1u << (4 * gfull)) - 1u);
  if (gfull < kBGroups) {
    const int nv = n - base - kBStep * gfull;
    vm |= (nv >= 4 ? 0xFu : (nv <= 0 ? 0u : (1u << nv) - 1u)) << (4 * gfull);
  }

  // A. load.  A NaN score is taken as -inf (its order is unspecified; this
  //    makes every comparison below a total preorder on floats, -0 == +0).
  //    Every position is loaded through a buffer resource bounded at the
  //    row's end, so a position past the end reads 0.  In the partly
  //    visible group row those zeros take part in the value range (which
  //    then covers 0 as well: still a valid range, at worst a coarser one);
  //    group rows wholly past the end are skipped by every per-item loop.
  //    Only the bin counts and the selection mask out the positions past
  //    the end.
#pragma unroll
  for (int k = 0; k < kBins / (4 * kBT); ++k)
    *reinterpret_cast<uint4*>(&sm.bins[4 * t + 4 * kBT * k]) = make_uint4(0u, 0u, 0u, 0u);
  if (t == 0) {
    lcount = 0;
    S.crowd = 0u;
    S.occ[0] = 0u;
    S.occ[1] = 0u;
  }
  // (adding +0 also turns -0 into +0, so the keys below need no fold)
  auto clean = [](float v) { return v == v ? v + 0.0f : -__builtin_inff(); };
  auto key_of = [](float v) {  // order_key for a value that is not -0
    const uint32_t u = __float_as_uint(v);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  };
  float x[kBPer];
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, n * 4, kRowBufWord3);
    // Group rows wholly inside the row (j < gfull, the same for every
    // thread) are read as one 16-byte load per thread when the row is
    // 16-byte aligned; the partly visible group row dword by dword, each
    // offset made opaque so that no two are merged into a multi-dword
    // access (whose bounds check need not be per dword); group rows past
    // the end hold zeros, as a load past the end would.
    const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
#pragma unroll
    for (int j = 0; j < kBGroups; ++j) {
      if (vec && j < gfull) {
        typedef uint32_t w4 __attribute__((ext_vector_type(4)));
        const w4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (base + kBStep * j), 0, 0);
        x[4 * j + 0] = __uint_as_float(v[0]);
        x[4 * j + 1] = __uint_as_float(v[1]);
        x[4 * j + 2] = __uint_as_float(v[2]);
        x[4 * j + 3] = __uint_as_float(v[3]);
      } else if (j < gused) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          int o = 4 * pos_of(4 * j + c);
          asm volatile("" : "+v"(o));
          x[4 * j + c] =
              __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0));
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[4 * j + c] = 0.0f;
      }
    }
  }
  float vlo = __builtin_inff(), vhi = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kBGroups; ++j) {
    if (j < gused) {  // (uniform) group rows past the end stay 0 and out of the range
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * j + c;
        x[i] = clean(x[i]);
        vlo = __builtin_fminf(vlo, x[i]);
        vhi = __builtin_fmaxf(vhi, x[i]);
      }
    }
  }
  {
    const uint32_t klo = __ockl_wfred_min_u32(order_key(vlo));
    const uint32_t khi = __ockl_wfred_max_u32(order_key(vhi));
    if (lane == 0) {
      fred[0][wid] = key_to_float(klo);
      fred[1][wid] = key_to_float(khi);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBT / 64; ++i) {
    vlo = __builtin_fminf(vlo, fred[0][i]);
    vhi = __builtin_fmaxf(vhi, fred[1][i]);
  }

  // Output of a chunk pass (after E, or at once when the chunk keeps
  //    everything): the selected set in ascending position order, with
  //    no order by score (only the last level orders).  A level's row is
  //    its chunks' lists back to back, each in ascending position, so
  //    position order is id order on every level, and the index-order tie
  //    break at T stays exact.  Slot = the items of lower group rows, plus
  //    those of lower threads in this group row, plus the lower lanes of
  //    this thread's float4: one block scan of the four per-group counts,
  //    packed 16 bits each (a group row holds at most 2048).
  auto chunk_out = [&](const uint32_t selm) {
    static_assert(!CHUNK || kBGroups == 4, "four group rows, two packed counts per scan word");
    auto gcount = [&](int j) { return __builtin_popcount((selm >> (4 * j)) & 0xFu); };
    int tot01, tot23;
    const int p01 = block_excl_scan<kBT>(gcount(0) | (gcount(1) << 16), red, &tot01);
    const int p23 = block_excl_scan<kBT>(gcount(2) | (gcount(3) << 16), red, &tot23);
    const int t0 = tot01 & 0xFFFF, t1 = tot01 >> 16, t2 = tot23 & 0xFFFF;
    const int gbase[4] = {p01 & 0xFFFF, t0 + (p01 >> 16), t0 + t1 + (p23 & 0xFFFF),
                          t0 + t1 + t2 + (p23 >> 16)};
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      if ((selm >> i) & 1u) {
        const int slot =
            gbase[i >> 2] + __builtin_popcount((selm >> (i & ~3)) & ((1u << (i & 3)) - 1u));
        const int p = pos_of(i);
        oi[slot] = idmap ? idmap[p] : (int32_t)(start + p);
        if (os) os[slot] = x[i];
      }
    }
    for (int q = cnt + t; q < K; q += kBT) {
      oi[q] = -1;
      if (os) os[q] = -__builtin_inff();
    }
  };
  if (CHUNK && !select) {  // a short chunk keeps all of it: no threshold
    chunk_out(vm);
    return;
  }

  // B. histogram over kBins bins linear in score value over [vmin, vmax]:
  //    bin(v) = (v - vmin) * scale rounded down, scale = (kBins - 0.01) /
  //    (vmax - vmin), so bin(vmax) < kBins after rounding.  bin() is
  //    monotone, so every item of a higher bin is greater than every item
  //    of a lower one.  A row without a finite positive span (all equal,
  //    infinities) puts everything in bin 0 and takes the general paths.
  //    (readfirstlane takes an int: broadcast the bit patterns.)
  const float vmin = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vlo)));
  const float vmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vhi)));
  const float span = vmax - vmin;
  const float scale0 = ((float)kBins - 0.01f) / span;
  const bool flat = !(span > 0.0f) || !(span <= 3.0e38f) || !(scale0 <= 3.0e38f);
  const float scale = flat ? 0.0f : scale0;
  const uint32_t keep_bins = flat ? 0u : 0xFFFFFFFFu;
  // the bins are computed once and kept packed, two per register
  uint32_t pk[kBPer / 2];
#pragma unroll
  for (int j = 0; j < kBPer / 2; ++j) {
    if (j / 2 < gused)
      pk[j] = ((uint32_t)((x[2 * j] - vmin) * scale) |
               ((uint32_t)((x[2 * j + 1] - vmin) * scale) << 16)) & keep_bins;
    else
      pk[j] = 0u;  // positions past the row: never counted or selected
  }
  auto bin_of = [&](int i) -> uint32_t { return (pk[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu; };
#pragma unroll
  for (int j = 0; j < kBGroups; ++j) {
    if (j < gfull) {
#pragma unroll
      for (int c = 0; c < 4; ++c) atomicAdd(&sm.bins[bin_of(4 * j + c)], 1u);
    } else if (j < gused) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((vm >> (4 * j + c)) & 1u) atomicAdd(&sm.bins[bin_of(4 * j + c)], 1u);
    }
  }
  __syncthreads();

  // C. b1 and the packed per-bin (offset << 16 | selected count), from the
  //    top; thread t owns the kBinsPer bins below kBins - kBinsPer t
  const int want = select ? K : n;
  int b1, ab1, in_bin;
  {
    const int top = kBins - 1 - kBinsPer * t;  // highest bin of this thread
    uint32_t c[kBinsPer];
#pragma unroll
    for (int v = 0; v < kBinsPer / 4; ++v) {
      const uint4 q = *reinterpret_cast<const uint4*>(&sm.bins[top - 3 - 4 * v]);
      c[4 * v + 0] = q.w;
      c[4 * v + 1] = q.z;
      c[4 * v + 2] = q.y;
      c[4 * v + 3] = q.x;
    }
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kBinsPer; ++j) sum += (int)c[j];
    int tot;
    const int ab = block_excl_scan<kBT>(sum, red, &tot);
    if (ab < want && ab + sum >= want) {
      int acc = ab;
#pragma unroll
      for (int j = 0; j < kBinsPer; ++j) {
        if (acc < want && acc + (int)c[j] >= want) {
          red[kBT / 64] = top - j;
          red[kBT / 64 + 1] = acc;
          red[kBT / 64 + 2] = (int)c[j];
        }
        acc += (int)c[j];
      }
    }
    __syncthreads();
    b1 = red[kBT / 64];
    ab1 = red[kBT / 64 + 1];
    in_bin = red[kBT / 64 + 2];
    // selected counts: all of every bin above b1, want - ab1 of b1; output
    // offsets are the exclusive prefix from the top (the ordering phases'
    // input: a chunk pass has none)
    if (!CHUNK) {
    uint32_t o = (uint32_t)ab, crowd = 0u;
#pragma unroll
    for (int j = 0; j < kBinsPer; ++j) {
      const int b = top - j;
      const uint32_t sel = b > b1 ? c[j] : (b == b1 ? (uint32_t)(want - ab1) : 0u);
      const uint32_t cj = c[j];
      c[j] = (o << 16) | sel;
      crowd = sel > crowd ? sel : crowd;
      o += cj;
    }
#pragma unroll
    for (int v = 0; v < kBinsPer / 4; ++v)
      *reinterpret_cast<uint4*>(&sm.bins[top - 3 - 4 * v]) =
          make_uint4(c[4 * v + 3], c[4 * v + 2], c[4 * v + 1], c[4 * v + 0]);
    crowd = __ockl_wfred_max_u32(crowd);
    if (lane == 0) atomicMax(&S.crowd, crowd);
    }
  }
  __syncthreads();
  const uint32_t crowd = CHUNK ? 0u : S.crowd;

  // D. the exact threshold value T inside b1
  float thr = 0.0f;
  int n_gt = 0, n_eq = 0;
  if (select) {
    const int need = K - ab1;  // rank of T among b1's items, >= 1
    // which of this thread's items lie in b1 (masks are built by doubling
    // and adding each compare, highest item first: one add per item)
    uint32_t inb = 0u;
#pragma unroll
    for (int i = kBPer - 1; i >= 0; --i)
      inb = (i >> 2) < gused ? inb + inb + (uint32_t)((int)bin_of(i) == b1) : inb + inb;
    inb &= vm;
    if (in_bin <= kBrute) {
      // b1 holds few items: each holder walks its set bits, re-reading the
      // score (a cached load, cleaned as in A) rather than indexing its
      // registers
      for (uint32_t mb = inb; mb != 0u; mb &= mb - 1u)
        sm.x.list[atomicAdd(&lcount, 1)] =
            __float_as_uint(clean(row[pos_of((int)__builtin_ctz(mb))]));
      __syncthreads();
      if (t < in_bin) {
        const float me = __uint_as_float(sm.x.list[t]);
        int g = 0, e = 0;
        for (int j = 0; j < in_bin; ++j) {
          const float v = __uint_as_float(sm.x.list[j]);
          g += v > me ? 1 : 0;
          e += v == me ? 1 : 0;
        }
        if (g < need && need <= g + e) {  // every holder of T writes the same values
          red[kBT / 64 + 3] = (int)__float_as_uint(me);
          red[kBT / 64 + 4] = g;
          red[kBT / 64 + 5] = e;
        }
      }
      __syncthreads();
      thr = __uint_as_float((uint32_t)red[kBT / 64 + 3]);
      n_gt = ab1 + red[kBT / 64 + 4];
      n_eq = red[kBT / 64 + 5];
    } else {
      // radix select among b1's items on the key digits 11/11/10; this rare
      // path re-reads b1's scores (from cache) rather than tying up the
      // register-resident row
      uint32_t prefix = 0u, pmask = 0u;
      int rank = need, above = ab1, count = in_bin;
#pragma unroll 1
      for (int level = 0; level < 3; ++level) {
        const int sh = level == 0 ? 21 : (level == 1 ? 10 : 0);
        const uint32_t dmask = level == 2 ? 1023u : 2047u;
        for (int i = t; i < 2048; i += kBT) sm.x.sub[i] = 0u;
        __syncthreads();
        asm volatile("" : "+v"(inb));
        for (uint32_t mb = inb; mb != 0u; mb &= mb - 1u) {
          const uint32_t k = order_key(clean(row[pos_of((int)__builtin_ctz(mb))]));
          if ((k & pmask) == prefix) atomicAdd(&sm.x.sub[(k >> sh) & dmask], 1u);
        }
        __syncthreads();
        int dig, ab;
        find_from_top<kBT>([&](int b) { return sm.x.sub[b]; }, 2048, rank, red, &dig, &ab,
                           &count);
        rank -= ab;
        above += ab;
        prefix |= (uint32_t)dig << sh;
        pmask |= dmask << sh;
      }
      thr = key_to_float(prefix);
      n_gt = above;
      n_eq = count;
    }
  }

  // E. selection: everything visible (no selection), or > T plus the
  //    need_eq lowest positions == T.  When T is tied beyond need_eq, the
  //    positions holding T go into a bitmap whose word prefix counts give
  //    each one its index-order rank among them.
  uint32_t selm = vm;
  if (select) {
    const int need_eq = K - n_gt;
    uint32_t gem = 0u;
#pragma unroll
    for (int i = kBPer - 1; i >= 0; --i)
      gem = (i >> 2) < gused ? gem + gem + (uint32_t)(x[i] >= thr) : gem + gem;
    selm = gem & vm;
    if (need_eq < n_eq) {  // uniform: T is tied past the K-th place
      uint32_t eqm = 0u;
#pragma unroll
      for (int i = kBPer - 1; i >= 0; --i)
        eqm = (i >> 2) < gused ? eqm + eqm + (uint32_t)(x[i] == thr) : eqm + eqm;
      eqm &= vm;
      const uint32_t gtm = selm & ~eqm;
      for (int i = t; i < kBN / 32; i += kBT) sm.x.eq.bits[i] = 0u;
      __syncthreads();
      // the four positions of group j share word (t >> 3) + 32 j
#pragma unroll
      for (int j = 0; j < kBGroups; ++j) {
        const uint32_t g4 = (eqm >> (4 * j)) & 0xFu;
        if (g4) atomicOr(&sm.x.eq.bits[(t >> 3) + (kBStep / 32) * j], g4 << (4 * (t & 7)));
      }
      __syncthreads();
      int tot;
      const uint32_t wbits = t < kBN / 32 ? sm.x.eq.bits[t] : 0u;
      const int wp = block_excl_scan<kBT>(__builtin_popcount(wbits), red, &tot);
      if (t < kBN / 32) sm.x.eq.pre[t] = (uint32_t)wp;
      __syncthreads();
      uint32_t keep = 0u;
#pragma unroll
      for (int i = 0; i < kBPer; ++i) {
        if ((eqm >> i) & 1u) {
          const int p = pos_of(i);
          const uint32_t w = sm.x.eq.bits[p >> 5];
          const int rank = (int)sm.x.eq.pre[p >> 5] + __builtin_popcount(w & ((1u << (p & 31)) - 1u));
          keep |= rank < need_eq ? (1u << i) : 0u;
        }
      }
      selm = gtm | keep;
      __syncthreads();  // the bitmap area is reused by the scatter
    }
  }

  if (CHUNK) {
    chunk_out(selm);
    return;
  }

  // F. scatter the selected items grouped by bin (cursor = packed high
  //    half), eight returning cursor atomics in flight, then their stores;
  //    the four entries past the last item are zeroed for the rank scan
  if (t < 4) sm.x.comp[cnt + t] = 0ull;
#pragma unroll
  for (int g = 0; g < kBGroups / 2; ++g) {
    if (2 * g < gused) {
      // (every item takes part, an unselected one on a word of its own lane
      // past the bins: with no branch around them the eight atomics are all
      // in flight before the first result is used)
      uint32_t slot[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = 8 * g + k;
        const uint32_t b = ((selm >> i) & 1u) ? bin_of(i) : (uint32_t)(kBins + (t & 63));
        slot[k] = atomicAdd(&sm.bins[b], 0x10000u);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = 8 * g + k;
        if ((selm >> i) & 1u) {
          // the key goes into a fresh register: the 64-bit store takes an
          // aligned pair, and a copy keeps the compiler from pinning all 32
          // items to pairs
          uint32_t kc;
          asm volatile("v_mov_b32 %0, %1" : "=v"(kc) : "v"(key_of(x[i])));
          const uint32_t lo = (bin_of(i) << kPosBits) | (kPosMask - (uint32_t)pos_of(i));
          sm.x.comp[slot[k] >> 16] = ((uint64_t)kc << 32) | lo;
        }
      }
    }
  }
  __syncthreads();

  // G+H. order and output.  Each selected item's slot is its bin's offset
  //    plus the number of same-bin items ahead of it under (score desc,
  //    index asc); items are written straight to that slot of the output
  //    row (a bin's items sit next to each other, so a wave's stores stay
  //    close to consecutive), and the slots past cnt get the padding.
  //    After the scatter a bin's packed word is ((offset + count) << 16 |
  //    count).  Positions are < n by construction; the clamp only keeps an
  //    id_map lookup in bounds.
  uint64_t occ = 0ull;
  auto emit = [&](int slot, uint64_t c) {
    uint32_t p = kPosMask - ((uint32_t)c & kPosMask);
    p = p < (uint32_t)n ? p : 0u;
    const int32_t id = idmap ? idmap[p] : (int32_t)(start + p);
    oi[slot] = id;
    if (os) os[slot] = key_to_float((uint32_t)(c >> 32));
    if (WIT && wL > 0) occ |= seg_bit(id, (uint32_t)wL, wS, wSe, wrcp);
  };
  if (crowd <= (uint32_t)kCrowd) {
#pragma unroll
    for (int m = 0; m < kBK / kBT; ++m) {
      const int q = t + kBT * m;
      if (q < cnt) {
        const uint64_t it = sm.x.comp[q];
        const uint32_t w = sm.bins[((uint32_t)it >> kPosBits) & (kBins - 1)];
        const uint32_t len = w & 0xFFFFu, s0 = (w >> 16) - len;
        const uint64_t* e = &sm.x.comp[s0];
        uint32_t rk = 0u;
        for (uint32_t jj = 0; jj < len; jj += 4) {
          rk += (uint32_t)(e[jj] > it) + (uint32_t)(e[jj + 1] > it) +
                (uint32_t)(e[jj + 2] > it) + (uint32_t)(e[jj + 3] > it);
        }
        emit((int)(s0 + rk), it);
      }
    }
  } else {
    const int P = next_pow2(cnt);
    for (int q = cnt + t; q < P; q += kBT) sm.x.comp[q] = 0ull;
    __syncthreads();
    bitonic_sort_desc<kBT>(sm.x.comp, P);
    for (int q = t; q < cnt; q += kBT) emit(q, sm.x.comp[q]);
  }
  for (int q = cnt + t; q < K; q += kBT) {
    oi[q] = -1;
    if (os) os[q] = -__builtin_inff();
  }
  if (wit && wL > 0) {  // the same for every thread of the row
    const uint32_t lo = __ockl_wfred_or_u32((uint32_t)occ);
    const uint32_t hi = __ockl_wfred_or_u32((uint32_t)(occ >> 32));
    if (lane == 0) {
      if (lo) atomicOr(&S.occ[0], lo);
      if (hi) atomicOr(&S.occ[1], hi);
    }
    // (the barrier also orders this row's output writes before the
    // witnesses that overwrite some of them)
    __syncthreads();
    if (wid == 0)
      write_witnesses(oi, ((uint64_t)S.occ[1] << 32) | S.occ[0], (uint32_t)wL, wSe, a.wit_keep,
                      a.wit_B);
  }
}

}  // namespace si
