// Decode-layout score micro-kernel pieces shared by the per-row score
// kernels and the prior-threshold path, so a key's score is the same bits
// whichever of them computes it.
#pragma once

#include "score_micro.hpp"

namespace si {

// Decode-layout fragments of row r: lane l supplies head mt * 32 + l % 32
// over its D-half, d = (D/2)(l/32) + 8 s + 0..7 in k-step s.
template <int MT, int KS>
__device__ __forceinline__ void load_rows_frags(const uint16_t* q, const float* w, int64_t w_stride,
                                                int r, int H, bf16x8 (&a)[1][MT][KS],
                                                float (&wv)[MT][16]) {
  constexpr int D = 16 * KS;
  const int lane = threadIdx.x & 63, hf = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int h = mt * 32 + (lane & 31);
    bool ok = h < H;
    const u32x4* src =
        reinterpret_cast<const u32x4*>(q + ((int64_t)r * H + (ok ? h : 0)) * D + hf * (D / 2));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = ok ? src[s] : u32x4{0u, 0u, 0u, 0u};
      a[0][mt][s] = as_bf16x8(x);
    }
  }
  load_w_frag<MT>(w, w_stride, r, H, true, wv);
}

// Score of this lane's key in a decode-layout 32-key tile: raw holds the
// lane's half-row (fp8 bytes, converted exactly to bf16, or bf16), sc the
// key's scale (fp8; applied after the head sum).  Every decode-layout path
// scores a key through this, so a key's score is the same bits on each.
template <int MT, int KS, bool FP8>
__device__ __forceinline__ float rows_tile_score(const bf16x8 (&a)[1][MT][KS],
                                                 const float (&wv)[MT][16],
                                                 const u32x4 (&raw)[FP8 ? KS / 2 : KS],
                                                 float sc) {
  f32x16 acc[1][MT];
  mfma_tiles<1, MT, KS>(
      a,
      [&](int s) {
        if (FP8) {
          u32x4 bb;
#pragma unroll
          for (int hw = 0; hw < 2; ++hw) {
            const uint32_t word = raw[s / 2][2 * (s % 2) + hw];
            auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
            auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true);
            bb[2 * hw + 0] = __builtin_bit_cast(uint32_t, p0);
            bb[2 * hw + 1] = __builtin_bit_cast(uint32_t, p1);
          }
          return as_bf16x8(bb);
        }
        return as_bf16x8(raw[s]);
      },
      acc);
  float s = head_reduce<MT>(acc[0], wv);
  if (FP8) s *= sc;
  return s;
}

// Optional score filter of the decode kernels: keep s >= tau[r]; each
// 32-key tile writes its survivor mask to bitmap[r * words + key / 32] and
// stores only the survivors' scores; each workgroup (row r, key chunk c)
// writes its survivor count to chunk_cnt[r * chunks + c].
struct RowsFilter {
  const float* tau;
  uint32_t* bitmap;
  int64_t words;
  int32_t* chunk_cnt;
  int64_t chunks;
};

// Each wave's survivor count of the workgroup's key chunk, at
// chunk_cnt[(r * chunks + chunk) * 4 + wave] (no barrier, so a wave that
// is done leaves at once).
__device__ __forceinline__ void filter_chunk_count(const RowsFilter& flt, int r, int count) {
  if ((threadIdx.x & 63) == 0)
    flt.chunk_cnt[((int64_t)r * flt.chunks + blockIdx.y) * 4 + (threadIdx.x >> 6)] = count;
}

}  // namespace si
