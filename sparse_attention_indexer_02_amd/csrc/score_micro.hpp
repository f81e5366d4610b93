// The bf16 MFMA score micro-kernel shared by every path that must produce
// the same bits for a (query, key) score: the prefill score kernel, and
// DoSA's seed scoring, survivor rescoring and exact fallback.
//
// Layout (v_mfma_f32_32x32x16_bf16): heads are MFMA rows, keys columns, D is
// the reduction.  Lane l supplies head row mt*32 + l%32 of the query and key
// column l%32; in k-step s both operands cover d = 16 s + 8 (l/32) + 0..7.
// The accumulator lane l holds rows 8*(v/4) + 4*(l/32) + v%4 (v = 0..15) of
// its key column.
#pragma once

#include "si_internal.hpp"

namespace si {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// max(x, 0) as one integer max on the bit pattern: every float with the sign
// bit set (negatives and -0) is a negative int32 and becomes +0.  Equal in
// value to fmaxf(x, 0) for every non-NaN x, without the NaN-quieting
// canonicalisation the IEEE-mode fmaxf costs.
__device__ __forceinline__ float relu(float x) {
  const int b = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, b > 0 ? b : 0);
}

// Waits for every outstanding memory operation of this wave.  Placed
// unconditionally before a key loop, it tells the compiler that the
// prologue's fragment loads have landed, so no wait on them (nor on the
// loop's own prefetch) is placed inside the loop.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Score epilogue: s = sum_h w_h max(x_h, 0) for this lane's key column.
// Fixed order: one fma chain per head tile mt over v = 0..15 in increasing
// v (two independent chains keep the VALU busy with MT = 2), the tiles'
// partials added in increasing mt, then lanes 0-31's partial is added to
// lanes 32-63's.  The order is part of what makes a score the same bits
// everywhere: every path that produces a (query, key) score calls this.
__device__ __forceinline__ float halves_sum(float s) {
  float o = __shfl_xor(s, 32, 64);
  return (threadIdx.x & 32) ? o + s : s + o;
}

template <int MT>
__device__ __forceinline__ float head_reduce(const f32x16 (&acc)[MT], const float (&wv)[MT][16]) {
  float p[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    p[mt] = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) p[mt] = __builtin_fmaf(wv[mt][v], relu(acc[mt][v]), p[mt]);
  }
  float s = p[0];
#pragma unroll
  for (int mt = 1; mt < MT; ++mt) s += p[mt];
  return halves_sum(s);
}

// Weight fragment of this lane for head tiles mt = 0..MT-1 of row r.
template <int MT>
__device__ __forceinline__ void load_w_frag(const float* w, int64_t w_stride, int r, int H,
                                            bool valid, float (&wv)[MT][16]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int h = mt * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      wv[mt][v] = (valid && h < H) ? w[(int64_t)r * w_stride + h] : 0.0f;
    }
}

// Query fragment of row r: head rows h = mt*32 + l%32 (zero beyond H).
template <int MT, int KS>
__device__ __forceinline__ void load_q_frag(const uint16_t* q, int r, int H, bool valid,
                                            bf16x8 (&a)[MT][KS]) {
  constexpr int D = 16 * KS;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int h = mt * 32 + (lane & 31);
    bool ok = valid && h < H;
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((int64_t)r * H + (ok ? h : 0)) * D);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = ok ? src[2 * s + (lane >> 5)] : u32x4{0u, 0u, 0u, 0u};
      a[mt][s] = as_bf16x8(v);
    }
  }
}

// acc[i] = query i's head tiles x one 32-key tile, for QPW queries sharing
// the key tile.  bfrag(s) returns this lane's 8 key elements of k-step s
// (d = 16 s + 8 (l/32) + 0..7 of key l%32).  Each accumulator sees the same
// MFMA sequence (k-steps in order from zero) whatever QPW is; k-step outer
// keeps QPW * MT independent chains in flight.
template <int QPW, int MT, int KS, class BFrag>
__device__ __forceinline__ void mfma_tiles(const bf16x8 (&a)[QPW][MT][KS], BFrag bfrag,
                                           f32x16 (&acc)[QPW][MT]) {
#pragma unroll
  for (int i = 0; i < QPW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][mt][v] = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    bf16x8 b = bfrag(s);
#pragma unroll
    for (int i = 0; i < QPW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[i][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][mt][s], b, acc[i][mt], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Key segments for the kernels that stream keys shared by all rows.  Keys
// beyond kSegThreshold bytes do not stay in one XCD's L2 while every resident
// workgroup streams all of them, so the launch is cut into 1 MiB key
// segments: workgroup b runs on XCD b % 8 (round-robin dispatch), and the
// XCDs walk the segments in step, each taking an eighth of the row groups
// (longest first unless the rows come from a list) for segment 0, then for
// segment 1, ..., so the workgroups resident on an XCD share one segment.
// ---------------------------------------------------------------------------
constexpr int64_t kSegBytes = 1 << 20;
constexpr int64_t kSegThreshold = 2 << 20;

// Segment count and keys per segment for `keys` shared keys of D bf16.
inline int key_segments(int64_t keys, int D, int64_t* seg_keys) {
  *seg_keys = kSegBytes / ((int64_t)D * 2);
  if (keys * D * 2 <= kSegThreshold) return 1;
  return (int)((keys + *seg_keys - 1) / *seg_keys);
}
// Workgroups to launch for G row groups.
inline int64_t segment_grid(int G, int nseg) {
  return nseg > 1 ? (int64_t)(G + 7) / 8 * 8 * nseg : G;
}
// This workgroup's row group and key range; false for a padding workgroup.
__device__ __forceinline__ bool segment_of(int G, int nseg, int64_t seg_keys, int64_t all_keys,
                                           bool longest_first, int* g, int64_t* lo,
                                           int64_t* hi) {
  if (nseg <= 1) {
    *g = longest_first ? G - 1 - (int)blockIdx.x : (int)blockIdx.x;
    *lo = 0;
    *hi = all_keys;
    return true;
  }
  const int G8 = (G + 7) / 8;  // groups per XCD per segment
  const int xcd = (int)(blockIdx.x % 8), seq = (int)(blockIdx.x / 8);
  const int seg = seq / G8, gi = xcd + 8 * (seq % G8);
  if (gi >= G) return false;
  *g = longest_first ? G - 1 - gi : gi;
  *lo = (int64_t)seg * seg_keys;
  *hi = *lo + seg_keys;
  return true;
}

}  // namespace si
