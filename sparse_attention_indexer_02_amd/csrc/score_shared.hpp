// The shared-key bf16 score loop of the prefill layout (the score stage's
// kernel is a thin wrapper around it).
#pragma once

#include "score_micro.hpp"

namespace si {

// Word 3 of a raw gfx9-family buffer resource: 32-bit data format, no
// swizzle, no index stride; with stride 0 the hardware range-checks the
// byte offset against num_records.
constexpr int kBufWord3 = 0x00020000;

// Bytes of LDS the score loop needs: two 32-key tiles of padded rows.
template <int KS>
constexpr int score_lds_bytes() {
  return 2 * 32 * (16 * KS * 2 + 16);
}

// Scores of the rows in slots g * 4 QPW .. of the workgroup (slot s -> row
// row_list ? row_list[s] : s, slots >= n_act empty) for the keys [key_lo,
// key_hi) (key_lo a multiple of 32), one wave per QPW of them: heads on the
// MFMA rows (32x32x16 bf16), keys on the columns, D the
// reduction; 32-key tiles of the shared keys are staged through LDS
// (double buffered) and read from L2 once per workgroup for all its rows;
// the ReLU * w head sum runs on the accumulator tile in registers.  lds is
// score_lds_bytes<KS>() of 16-byte aligned shared memory.  Every thread of
// the workgroup must call it.
template <int MT, int KS, int QPW>
__device__ __forceinline__ void score_group_shared(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int64_t w_stride, const int32_t* __restrict__ vis_len, int H, int64_t n_k, int64_t max_vis,
    float* __restrict__ scores, int64_t score_stride, const int32_t* __restrict__ row_list,
    int n_act, int g, int64_t key_lo, int64_t key_hi, unsigned char* lds_base) {
  constexpr int D = 16 * KS;
  constexpr int QB = 4 * QPW;                  // queries per workgroup
  constexpr int ROWB = D * 2 + 16;             // padded LDS row: conflict-free b128 reads
  constexpr int CPK = D * 2 / 16;              // 16-byte chunks per key
  constexpr int CHUNKS = 32 * CPK;             // 16-byte chunks per 32-key tile
  constexpr int CPT = (CHUNKS + 255) / 256;    // chunks per thread
  unsigned char (*lds)[32 * ROWB] = reinterpret_cast<unsigned char (*)[32 * ROWB]>(lds_base);

  const int lane = threadIdx.x & 63, wave = wave_index();
  auto row_of = [&](int i) -> int {  // slot i of this workgroup -> row, or -1
    int s = g * QB + i;
    if (s >= n_act) return -1;
    return row_list ? row_list[s] : s;
  };

  int myrow[QPW];
  int64_t vis[QPW];
  int64_t end = 0;  // keys any row of the group sees
  for (int i = 0; i < QB; ++i) {
    int r = row_of(i);
    int64_t off, v = 0;
    if (r >= 0) v = visible_len(vis_len, nullptr, r, n_k, max_vis, &off);
    end = v > end ? v : end;
    if (i / QPW == wave) {
      vis[i % QPW] = v;
      myrow[i % QPW] = r;
    }
  }
  end = end < key_hi ? end : key_hi;
  if (end <= key_lo) return;

  bf16x8 a[QPW][MT][KS];
  float wv[QPW][MT][16];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    load_q_frag<MT, KS>(q, myrow[i], H, myrow[i] >= 0, a[i]);
    load_w_frag<MT>(w, w_stride, myrow[i], H, myrow[i] >= 0, wv[i]);
  }

  const int t_lo = (int)(key_lo / 32), ntiles = (int)((end + 31) / 32);
  u32x4 pre[CPT];
  static_assert(CHUNKS % 256 == 0, "every thread stages whole chunks");
  // Keys and score rows go through buffer resources: 32-bit offsets (one
  // VALU op per address) and the hardware range check, which returns zero
  // for a key load past n_k and drops a score store past the row's visible
  // length, so no load or store sits under a branch and the compiler keeps
  // every memory wait out of the MFMA section.  The launcher guarantees
  // n_k * D * 2 < 2^31.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)k, (short)0, (int)(n_k * D * 2), kBufWord3);
  __amdgpu_buffer_rsrc_t srs[QPW];
#pragma unroll
  for (int i = 0; i < QPW; ++i)
    srs[i] = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(scores + (int64_t)(myrow[i] >= 0 ? myrow[i] : 0) * score_stride), (short)0,
        (int)(myrow[i] >= 0 ? vis[i] * 4 : 0), kBufWord3);
  auto fetch = [&](int t) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      pre[c] = __builtin_amdgcn_raw_buffer_load_b128(krs, t * (32 * D * 2) + (threadIdx.x + 256 * c) * 16,
                                                     0, 0);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = threadIdx.x + 256 * c;
      const int key = ch / CPK, part = ch % CPK;
      *reinterpret_cast<u32x4*>(&lds[buf][key * ROWB + part * 16]) = pre[c];
    }
  };
  const unsigned char* lrow = &lds[0][(lane & 31) * ROWB + (lane >> 5) * 16];

  fetch(t_lo);
  stash(t_lo & 1);
  wait_memory();
  __syncthreads();
  for (int t = t_lo; t < ntiles; ++t) {
    fetch(t + 1 < ntiles ? t + 1 : t);  // the last one is a harmless repeat
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
    const unsigned char* brow = lrow + (t & 1) * (32 * ROWB);
    f32x16 acc[QPW][MT];
    mfma_tiles<QPW, MT, KS>(
        a, [&](int s) { return as_bf16x8(*reinterpret_cast<const u32x4*>(brow + 32 * s)); },
        acc);
    float sc[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) sc[i] = head_reduce<MT>(acc[i], wv[i]);
    // the stash waits for the prefetch: keep it after the head sums, so the
    // load has the whole tile's MFMAs and epilogue to land
    __builtin_amdgcn_sched_barrier(0);
    // buffer (t + 1) & 1 held tile t - 1, read before the previous barrier
    stash((t + 1) & 1);
    // lanes 32-63 hold the same sums; their out-of-range offset drops them
    const int off = lane < 32 ? (t * 32 + lane) * 4 : INT32_MAX;
#pragma unroll
    for (int i = 0; i < QPW; ++i)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc[i]), srs[i], off, 0, 0);
    __syncthreads();
  }
}

}  // namespace si
