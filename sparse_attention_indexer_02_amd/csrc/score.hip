// Lightning-indexer score  s[r, j] = sum_h w[r, h] * max(q[r, h, :] . k[j, :], 0)
// (DoSA reading notes, section 3), written for every visible key.
//
// Kernels:
//  * score_mfma_shared: bf16 q and bf16 keys shared by all rows (prefill).
//    Heads sit in the MFMA row dimension (32x32x16 bf16 tiles), keys in
//    the column dimension, D is the reduction.  A workgroup of 4 waves owns
//    4*QPW queries and streams 32-key tiles through LDS (double buffered);
//    each key tile is read from L2 once per workgroup and feeds every query
//    of it.  The ReLU * w head reduction runs in registers on the
//    accumulator tile.  Optionally driven by a device row list.
//  * score_mfma_rows: bf16 queries against bf16 per-row keys (decode
//    layout).  No reuse across rows, so keys go straight to registers.
//  * score_mfma_rows_fp8: the same with OCP fp8 e4m3fn keys, staged through
//    a per-wave LDS ring and converted exactly to bf16; the per-token scale
//    is applied after the head sum (ReLU(c x) = c ReLU(x) for c > 0).
//    Optionally filters the written scores by a per-row threshold.
//  * score_mfma_f32: fp32 queries and keys on v_mfma_f32_32x32x2_f32 with
//    the same accumulator layout and head sum.
//  * score_generic: VALU fp32 path for the shapes and dtype mixes the MFMA
//    kernels do not cover.
#include "score_rows.hpp"
#include "score_shared.hpp"

namespace si {

// ---------------------------------------------------------------------------
// Shared-key prefill kernel: one workgroup per 4 QPW rows and key segment
// (segments as in score_micro.hpp; one segment when the keys fit an L2).
// ---------------------------------------------------------------------------
template <int MT, int KS, int QPW>
__global__ __launch_bounds__(256, 2) void score_mfma_shared(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int64_t w_stride, const int32_t* __restrict__ vis_len, int n_q, int H, int64_t n_k,
    int64_t max_vis, float* __restrict__ scores, int64_t score_stride,
    const int32_t* __restrict__ row_list, const int32_t* __restrict__ row_count, int nseg,
    int64_t seg_keys) {
  constexpr int QB = 4 * QPW;
  __shared__ __attribute__((aligned(16))) unsigned char lds[score_lds_bytes<KS>()];
  const int n_act = row_list ? *row_count : n_q;
  const int G = (n_q + QB - 1) / QB;  // groups the grid was sized for
  int g;
  int64_t key_lo, key_hi;
  // listed rows keep list order; otherwise longest rows (highest index) first
  if (!segment_of(G, nseg, seg_keys, max_vis, row_list == nullptr, &g, &key_lo, &key_hi)) return;
  if (g * QB >= n_act) return;
  score_group_shared<MT, KS, QPW>(q, k, w, w_stride, vis_len, H, n_k, max_vis, scores,
                                  score_stride, row_list, n_act, g, key_lo, key_hi, lds);
}

// ---------------------------------------------------------------------------
// Per-row keys (decode layout), bf16 or fp8 keys.  Grid (rows, chunks); each
// wave takes the 32-key tiles wave, wave + 4, ... of its row's chunk.  Lane l
// handles key l%32 and the D-half l/32: in k-step s it supplies d =
// (D/2)(l/32) + 8 s + 0..7, so each lane reads one contiguous half-row; the
// query fragments use the same d order.  The keys go straight to registers
// (no reuse across rows), one tile ahead of the MFMAs, through buffer
// resources bounded at the chunk's end (loads past it read zero, stores past
// it are dropped), so neither loads nor stores sit under a branch.
// ---------------------------------------------------------------------------

template <int MT, int KS, bool FP8, bool FILT>
__global__ __launch_bounds__(256, 2) void score_mfma_rows(
    const uint16_t* __restrict__ q, const void* __restrict__ kv, const float* __restrict__ kscale,
    const float* __restrict__ w, int64_t w_stride, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ vis_len, int n_q, int H, int64_t n_k, int64_t max_vis,
    float* __restrict__ scores, int64_t score_stride, RowsFilter flt) {
  constexpr int D = 16 * KS;
  constexpr int ES = FP8 ? 1 : 2;        // bytes per key element
  constexpr int NL = FP8 ? KS / 2 : KS;  // 16-byte loads per lane per tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = rows_grid_row();
  int64_t off;
  const int64_t v = visible_len(vis_len, row_off, r, n_k, max_vis, &off);
  const int64_t c0 = (int64_t)blockIdx.y * kRowsChunk;
  if (c0 >= v) return;
  const int nk = (int)((c0 + kRowsChunk < v) ? kRowsChunk : v - c0);

  bf16x8 a[1][MT][KS];
  float wv[MT][16];
  load_rows_frags<MT, KS>(q, w, w_stride, r, H, a, wv);
  const float tr = FILT ? flt.tau[r] : 0.0f;
  int kept = 0;  // survivors this wave stored (filter only)

  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(kv) + (off + c0) * D * ES), (short)0, nk * D * ES,
      kBufWord3);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(FP8 ? kscale + off + c0 : kscale), (short)0, FP8 ? nk * 4 : 0, kBufWord3);
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scores + (int64_t)r * score_stride + c0), (short)0, nk * 4, kBufWord3);
  const int lk = lane & 31;
  const int lane_off = lk * D * ES + (lane >> 5) * (D / 2) * ES;

  auto load = [&](int tt, u32x4 (&raw)[NL], float& sc) {
    const int o = tt * D * ES + lane_off;
#pragma unroll
    for (int c = 0; c < NL; ++c) raw[c] = __builtin_amdgcn_raw_buffer_load_b128(krs, o + 16 * c, 0, 0);
    sc = FP8 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(crs, (tt + lk) * 4, 0, 0))
             : 1.0f;
  };
  auto compute = [&](int tt, const u32x4 (&raw)[NL], float sc) {
    const float s = rows_tile_score<MT, KS, FP8>(a, wv, raw, sc);
    // lanes 32-63 hold the same sums; their out-of-range offset drops them
    int o = lane < 32 ? (tt + lane) * 4 : INT32_MAX;
    if (FILT) {
      const bool keep = lane < 32 && tt + lane < nk && s >= tr;
      const uint64_t m = __ballot(keep);
      if (lane == 0 && tt < nk) flt.bitmap[(int64_t)r * flt.words + ((c0 + tt) >> 5)] = (uint32_t)m;
      kept += __builtin_popcountll(m);
      o = keep ? o : INT32_MAX;
    }
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s), ors, o, 0, 0);
  };

  // tiles wave * 32 + 128 i, i < n_i; two register sets alternate so the
  // next tile's loads are in flight during each tile's MFMAs
  const int first = wave * 32;
  const int n_i = first < nk ? (nk - first + 127) / 128 : 0;
  u32x4 ra[NL], rb[NL];
  float sa = 0.0f, sb = 0.0f;
  if (n_i > 0) load(first, ra, sa);
  int i = 0;
  for (; i + 1 < n_i; i += 2) {
    load(first + 128 * (i + 1), rb, sb);
    compute(first + 128 * i, ra, sa);
    load(first + 128 * (i + 2), ra, sa);  // past the chunk: reads zero, never used
    compute(first + 128 * (i + 1), rb, sb);
  }
  if (i < n_i) compute(first + 128 * i, ra, sa);
  if (FILT) filter_chunk_count(flt, r, kept);
}

// ---------------------------------------------------------------------------
// Per-row fp8 keys (decode layout), staged through LDS by the buffer unit.
// Same lane roles and arithmetic as score_mfma_rows<.., true>; each wave owns
// a ring of kRingTiles tile buffers in LDS that the buffer loads fill
// directly (no registers held for the prefetch), kRingTiles - 1 tiles ahead
// of the MFMAs, so several tiles per wave are in flight.  A tile's 16-byte
// chunks are placed at slot k * CPK + (c ^ f(k)) (key k, chunk c, f(k) =
// (k % 8) ^ ((k / 8) % 2), taken mod CPK), so the MFMA-order reads (lanes =
// keys, same chunk) of 8 or 16 consecutive keys hit distinct 16-byte bank
// groups whether one LDS cycle serves 128 or 256 bytes; the loader lanes
// cover 8 whole keys per instruction.  The key scales ride
// along (one dword per key).  A wave only ever reads its own ring, so the
// waits are the wave's own load counter, no barrier.  Loads past the chunk
// are clamped to its last key.
// ---------------------------------------------------------------------------
constexpr int kRingTiles = 3;

// LDS byte address of a shared-memory object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// One buffer-unit load straight into LDS: 16 (or 4) bytes per lane from the
// lane's global address into lds + 16 (or 4) * lane.  Written as assembly so
// that the compiler's own wait placement does not treat every later LDS
// read as depending on it; the kernel waits on the load counter itself.
__device__ __forceinline__ void lds_load16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

template <int MT, int KS, bool FILT>
__global__ __launch_bounds__(256, 3) void score_mfma_rows_fp8(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
    const float* __restrict__ kscale, const float* __restrict__ w, int64_t w_stride,
    const int64_t* __restrict__ row_off, const int32_t* __restrict__ vis_len, int n_q, int H,
    int64_t n_k, int64_t max_vis, float* __restrict__ scores, int64_t score_stride,
    RowsFilter flt) {
  constexpr int D = 16 * KS;
  constexpr int CPK = D / 16;      // 16-byte chunks per key
  constexpr int TB = 32 * D;       // bytes per 32-key tile
  constexpr int NDMA = TB / 1024;  // 64-lane x 16-byte loads per tile
  constexpr int NB = kRingTiles;
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[4][NB][TB];
  __shared__ __attribute__((aligned(16))) float sbuf[4][NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = rows_grid_row();
  int64_t off;
  const int64_t v = visible_len(vis_len, row_off, r, n_k, max_vis, &off);
  const int64_t c0 = (int64_t)blockIdx.y * kRowsChunk;
  if (c0 >= v) return;
  const int nk = (int)((c0 + kRowsChunk < v) ? kRowsChunk : v - c0);

  const int first = wave * 32;
  const int n_i = first < nk ? (nk - first + 127) / 128 : 0;
  // this lane's share of a tile load: slot p = 64 d + lane holds key p / CPK,
  // chunk (p % CPK) ^ (key % CPK)
  auto swz = [](int k) { return ((k & 7) ^ ((k >> 3) & 1)) % CPK; };
  int gkey[NDMA], gch[NDMA];
#pragma unroll
  for (int d = 0; d < NDMA; ++d) {
    const int p = 64 * d + lane;
    gkey[d] = p / CPK;
    gch[d] = (p % CPK) ^ swz(gkey[d]);
  }
  const uint8_t* kc = kv + (off + c0) * D;
  const float* sc0 = kscale + off + c0;
  // ring tile i of this wave = keys first + 128 i ..; a key past the chunk
  // is read as the chunk's last key (its score is never stored)
  const uint32_t kring = __builtin_amdgcn_readfirstlane(lds_addr(&kbuf[wave][0][0]));
  const uint32_t sring = __builtin_amdgcn_readfirstlane(lds_addr(&sbuf[wave][0][0]));
  auto issue = [&](int i) {
    const int tt = first + 128 * i, b = i % NB;
#pragma unroll
    for (int d = 0; d < NDMA; ++d) {
      const int key = tt + gkey[d] < nk ? tt + gkey[d] : nk - 1;
      lds_load16(kc + (int64_t)key * D + gch[d] * 16, kring + b * TB + 1024 * d);
    }
    const int key = tt + lane < nk ? tt + lane : nk - 1;
    lds_load4(sc0 + key, sring + b * 256);
  };
  const int lk = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) issue(i);
  bf16x8 a[1][MT][KS];
  float wv[MT][16];
  load_rows_frags<MT, KS>(q, w, w_stride, r, H, a, wv);
  const float tr = FILT ? flt.tau[r] : 0.0f;
  int kept = 0;  // survivors this wave stored (filter only)
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scores + (int64_t)r * score_stride + c0), (short)0, nk * 4, kBufWord3);

  for (int i = 0; i < n_i; ++i) {
    // the buffer refilled here was read in step i - 1, whose reads have
    // been consumed
    __builtin_amdgcn_sched_barrier(0);
    issue(i + NB - 1);
    // tile i's loads are complete once at most the later tiles' loads
    // (issued after it, and returned in order) are outstanding
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NB - 1) * (NDMA + 1)) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* tb = &kbuf[wave][i % NB][0];
    u32x4 ch[CPK / 2];
#pragma unroll
    for (int j = 0; j < CPK / 2; ++j) {
      const int c = hf * (CPK / 2) + j;
      ch[j] = *reinterpret_cast<const u32x4*>(tb + 16 * (lk * CPK + (c ^ swz(lk))));
    }
    const float sc = sbuf[wave][i % NB][lk];
    const float s = rows_tile_score<MT, KS, true>(a, wv, ch, sc);
    // lanes 32-63 hold the same sums; their out-of-range offset drops them
    const int tt = first + 128 * i;
    int o = lane < 32 ? (tt + lane) * 4 : INT32_MAX;
    if (FILT) {
      const bool keep = lane < 32 && tt + lane < nk && s >= tr;
      const uint64_t m = __ballot(keep);
      if (lane == 0 && tt < nk) flt.bitmap[(int64_t)r * flt.words + ((c0 + tt) >> 5)] = (uint32_t)m;
      kept += __builtin_popcountll(m);
      o = keep ? o : INT32_MAX;
    }
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s), ors, o, 0, 0);
  }
  // no load may still be writing this wave's ring when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (FILT) filter_chunk_count(flt, r, kept);
}

// ---------------------------------------------------------------------------
// Generic VALU path: one thread per (row, key), fp32 arithmetic.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float decode_elem(const void* p, si_dtype dt, int64_t i) {
  if (dt == SI_F32) return reinterpret_cast<const float*>(p)[i];
  if (dt == SI_BF16)
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
  uint32_t b = reinterpret_cast<const uint8_t*>(p)[i];
  // OCP e4m3fn: place exponent/mantissa in an f32 and rescale by 2^120
  // (exact, subnormals included); S.1111.111 is NaN.
  if ((b & 0x7Fu) == 0x7Fu) return __uint_as_float(0x7FC00000u | ((b & 0x80u) << 24));
  float mag = __uint_as_float((b & 0x7Fu) << 20) * 0x1p120f;
  return (b & 0x80u) ? -mag : mag;
}

constexpr int kGenericMaxQ = 8192;  // H * D floats held in LDS

__global__ __launch_bounds__(256) void score_generic(ScoreArgs a) {
  __shared__ float qs[kGenericMaxQ];
  __shared__ float ws[1024];
  const int r = blockIdx.x;
  const int H = a.H, D = a.D;
  for (int i = threadIdx.x; i < H * D; i += 256)
    qs[i] = decode_elem(a.q, a.q_dtype, (int64_t)r * H * D + i);
  for (int i = threadIdx.x; i < H; i += 256) ws[i] = a.w[(int64_t)r * a.w_row_stride + i];
  __syncthreads();
  int64_t off;
  const int64_t v = visible_len(a.vis_len, a.k_row_offset, r, a.n_k, a.max_vis, &off);
  const int64_t j = (int64_t)blockIdx.y * 256 + threadIdx.x;
  if (j >= v) return;
  const int64_t key = off + j;
  float s = 0.0f;
  for (int h0 = 0; h0 < H; h0 += 16) {
    float x[16];
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) x[hh] = 0.0f;
    for (int d = 0; d < D; ++d) {
      float kd = decode_elem(a.k, a.k_dtype, key * D + d);
#pragma unroll
      for (int hh = 0; hh < 16; ++hh)
        if (h0 + hh < H) x[hh] = __builtin_fmaf(qs[(h0 + hh) * D + d], kd, x[hh]);
    }
#pragma unroll
    for (int hh = 0; hh < 16; ++hh)
      if (h0 + hh < H) s = __builtin_fmaf(ws[h0 + hh], __builtin_fmaxf(x[hh], 0.0f), s);
  }
  if (a.k_dtype == SI_FP8_E4M3FN) s *= a.k_scale[key];
  a.scores[(int64_t)r * a.score_stride + j] = s;
}

// ---------------------------------------------------------------------------
// fp32 queries and keys: v_mfma_f32_32x32x2_f32 tiles with the same roles as
// the bf16 path (heads on the MFMA rows, 32 keys on the columns, two d per
// step: lane l supplies head l % 32, or key l % 32, at d = 2 s + l / 32),
// and the same ReLU * w head sum (head_reduce), which the 32x32 accumulator
// layout shares.  One wave per 32-key tile, four tiles of a row per
// workgroup; the query fragments are read from the cache per step.
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(256) void score_mfma_f32(ScoreArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = rows_grid_row();
  int64_t off;
  const int64_t v = visible_len(a.vis_len, a.k_row_offset, r, a.n_k, a.max_vis, &off);
  const int64_t t0 = ((int64_t)blockIdx.y * 4 + wave) * 32;  // this wave's first key
  if (t0 >= v) return;
  const int H = a.H, D = a.D, hk = lane >> 5;
  const int64_t key = t0 + (lane & 31);
  const bool kvis = key < v;
  // a key past the row is read as the tile's first key; its score is not stored
  const float* krow = reinterpret_cast<const float*>(a.k) + (off + (kvis ? key : t0)) * D;
  const float* qrow = reinterpret_cast<const float*>(a.q) + (int64_t)r * H * D;
  float wv[MT][16];
  load_w_frag<MT>(a.w, a.w_row_stride, r, H, true, wv);
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mt][e] = 0.0f;
  for (int d = 0; d < D; d += 2) {
    const float b = krow[d + hk];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 32 + (lane & 31);
      const float av = h < H ? qrow[(int64_t)h * D + d + hk] : 0.0f;
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b, acc[mt], 0, 0, 0);
    }
  }
  const float s = head_reduce<MT>(acc, wv);
  if (lane < 32 && kvis) a.scores[(int64_t)r * a.score_stride + key] = s;
}

// ---------------------------------------------------------------------------
// Dispatch.
// ---------------------------------------------------------------------------
bool score_mfma_supported(const ScoreArgs& a) {
  if (a.q_dtype != SI_BF16) return false;
  if (a.k_dtype != SI_BF16 && a.k_dtype != SI_FP8_E4M3FN) return false;
  if (a.D != 64 && a.D != 128) return false;
  return a.H >= 1 && a.H <= 64;
}

template <int MT, int KS>
static hipError_t launch_mfma(const ScoreArgs& a, const int32_t* row_list,
                              const int32_t* row_count, hipStream_t st) {
  // shared bf16 keys small enough for 32-bit buffer offsets go through the
  // LDS-sharing kernel; listed rows exist only on that path
  const bool shared = a.k_row_offset == nullptr && a.k_dtype == SI_BF16 &&
                      a.n_k * a.D * 2 <= (int64_t)INT32_MAX &&
                      a.max_vis * 4 <= (int64_t)INT32_MAX;
  if (row_list != nullptr && !shared) return hipErrorInvalidValue;
  if (a.filter_tau != nullptr &&
      (shared || a.filter_bitmap == nullptr || a.filter_chunk_cnt == nullptr))
    return hipErrorInvalidValue;  // decode layout only, with both outputs
  if (shared) {
    constexpr int QPW = (MT == 1) ? 2 : 1;
    const int groups = (a.n_q + 4 * QPW - 1) / (4 * QPW);
    int64_t seg_keys;
    const int nseg = key_segments(a.max_vis < a.n_k ? a.max_vis : a.n_k, a.D, &seg_keys);
    const int64_t grid = segment_grid(groups, nseg);
    hipLaunchKernelGGL((score_mfma_shared<MT, KS, QPW>), dim3((unsigned)grid), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(a.q),
                       reinterpret_cast<const uint16_t*>(a.k), a.w, a.w_row_stride, a.vis_len,
                       a.n_q, a.H, a.n_k, a.max_vis, a.scores, a.score_stride, row_list,
                       row_count, nseg, seg_keys);
  } else {
    const int64_t chunks = (a.max_vis + kRowsChunk - 1) / kRowsChunk;
    dim3 grid((unsigned)a.n_q, (unsigned)(chunks > 0 ? chunks : 1));
    const RowsFilter flt{a.filter_tau, a.filter_bitmap, a.filter_words, a.filter_chunk_cnt,
                         chunks};
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(a.q);
    if (a.k_dtype == SI_FP8_E4M3FN) {
      const uint8_t* k8 = reinterpret_cast<const uint8_t*>(a.k);
      if (flt.tau)
        hipLaunchKernelGGL((score_mfma_rows_fp8<MT, KS, true>), grid, dim3(256), 0, st, q16, k8,
                           a.k_scale, a.w, a.w_row_stride, a.k_row_offset, a.vis_len, a.n_q, a.H,
                           a.n_k, a.max_vis, a.scores, a.score_stride, flt);
      else
        hipLaunchKernelGGL((score_mfma_rows_fp8<MT, KS, false>), grid, dim3(256), 0, st, q16, k8,
                           a.k_scale, a.w, a.w_row_stride, a.k_row_offset, a.vis_len, a.n_q, a.H,
                           a.n_k, a.max_vis, a.scores, a.score_stride, flt);
    } else {
      if (flt.tau)
        hipLaunchKernelGGL((score_mfma_rows<MT, KS, false, true>), grid, dim3(256), 0, st, q16,
                           a.k, a.k_scale, a.w, a.w_row_stride, a.k_row_offset, a.vis_len, a.n_q,
                           a.H, a.n_k, a.max_vis, a.scores, a.score_stride, flt);
      else
        hipLaunchKernelGGL((score_mfma_rows<MT, KS, false, false>), grid, dim3(256), 0, st, q16,
                           a.k, a.k_scale, a.w, a.w_row_stride, a.k_row_offset, a.vis_len, a.n_q,
                           a.H, a.n_k, a.max_vis, a.scores, a.score_stride, flt);
    }
  }
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  if (a.n_q == 0 || a.max_vis == 0) return hipSuccess;
  if (score_mfma_supported(a)) {
    const int MT = a.H <= 32 ? 1 : 2;
    if (a.D == 128)
      return MT == 1 ? launch_mfma<1, 8>(a, nullptr, nullptr, st)
                     : launch_mfma<2, 8>(a, nullptr, nullptr, st);
    return MT == 1 ? launch_mfma<1, 4>(a, nullptr, nullptr, st)
                   : launch_mfma<2, 4>(a, nullptr, nullptr, st);
  }
  if (a.q_dtype == SI_F32 && a.k_dtype == SI_F32 && a.D % 2 == 0 && a.H >= 1 && a.H <= 64) {
    const int64_t by = (a.max_vis + 127) / 128;  // four 32-key tiles per workgroup
    const dim3 grid((unsigned)a.n_q, (unsigned)by);
    if (a.H <= 32) hipLaunchKernelGGL(score_mfma_f32<1>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(score_mfma_f32<2>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int64_t bx = (a.max_vis + 255) / 256;
  hipLaunchKernelGGL(score_generic, dim3((unsigned)a.n_q, (unsigned)bx), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Shared-key bf16 scoring of the rows listed on the device (row_list[0 ..
// *row_count)), with exactly the arithmetic of launch_score for the same
// shapes; n_q bounds the list length.
hipError_t launch_score_rows_listed(const ScoreArgs& a, const int32_t* row_list,
                                    const int32_t* row_count, hipStream_t st) {
  if (a.n_q == 0 || a.max_vis == 0) return hipSuccess;
  const int MT = a.H <= 32 ? 1 : 2;
  if (a.D == 128)
    return MT == 1 ? launch_mfma<1, 8>(a, row_list, row_count, st)
                   : launch_mfma<2, 8>(a, row_list, row_count, st);
  return MT == 1 ? launch_mfma<1, 4>(a, row_list, row_count, st)
                 : launch_mfma<2, 4>(a, row_list, row_count, st);
}

}  // namespace si
