// Segment-witness merge, in place ("Segment Witnesses" page: Object,
// Implementation rule and contracts).
//
// One wave per row.  Lanes stream the row with 16-byte loads and OR each
// entry's segment bit (witness_seg.hpp) into a 64-bit occupancy mask; the
// mask is OR-reduced across the wave; lane s (< S_eff) then owns segment s:
// if it is empty its witness e_s = ceil(s L / S_eff) takes slot keep +
// (number of empty segments below s), when that rank is < B.  Only those
// <= B slots are written.
#include "witness_seg.hpp"

namespace si {

constexpr int kWitThreads = 256;

__global__ __launch_bounds__(kWitThreads) void witness_merge(int32_t* __restrict__ idx, int rows,
                                                             int topk,
                                                             const int32_t* __restrict__ lens,
                                                             int S, int keep, int B) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (kWitThreads / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int32_t Ls = lens[r];
  if (Ls <= 0) return;  // no witnesses for an empty or negative context
  const uint32_t L = (uint32_t)Ls;
  const uint32_t Se = (uint32_t)S < L ? (uint32_t)S : L;
  const float rcpL = 1.0f / (float)L;
  int32_t* row = idx + (int64_t)r * topk;

  uint64_t occ = 0ull;
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  int t0 = 0;
  if (vec && L < (1u << 26)) {
    // 16-byte loads, four rounds of loads in flight before their use
    const int nv = topk >> 2;
    const int4* rv = reinterpret_cast<const int4*>(row);
    int i = lane;
    for (; i + 192 < nv; i += 256) {
      int4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = rv[i + 64 * u];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        occ |= seg_bit32(x[u].x, L, S, Se, rcpL) | seg_bit32(x[u].y, L, S, Se, rcpL) |
               seg_bit32(x[u].z, L, S, Se, rcpL) | seg_bit32(x[u].w, L, S, Se, rcpL);
    }
    for (; i < nv; i += 64) {
      const int4 x = rv[i];
      occ |= seg_bit32(x.x, L, S, Se, rcpL) | seg_bit32(x.y, L, S, Se, rcpL) |
             seg_bit32(x.z, L, S, Se, rcpL) | seg_bit32(x.w, L, S, Se, rcpL);
    }
    t0 = nv << 2;
  } else if (vec) {
    const int nv = topk >> 2;
    const int4* rv = reinterpret_cast<const int4*>(row);
    for (int i = lane; i < nv; i += 64) {
      int4 x = rv[i];
      occ |= seg_bit(x.x, L, S, Se, rcpL) | seg_bit(x.y, L, S, Se, rcpL) |
             seg_bit(x.z, L, S, Se, rcpL) | seg_bit(x.w, L, S, Se, rcpL);
    }
    t0 = nv << 2;
  }
  for (int t = t0 + lane; t < topk; t += 64) occ |= seg_bit(row[t], L, S, Se, rcpL);
  occ = ((uint64_t)__ockl_wfred_or_u32((uint32_t)(occ >> 32)) << 32) |
        __ockl_wfred_or_u32((uint32_t)occ);
  write_witnesses(row, occ, L, Se, keep, B);
}

hipError_t launch_witness(int32_t* idx, int32_t rows, int32_t topk, const int32_t* lens,
                          int32_t S, int32_t keep, int32_t B, hipStream_t st) {
  const int per = kWitThreads / 64;
  hipLaunchKernelGGL(witness_merge, dim3((unsigned)((rows + per - 1) / per)), dim3(kWitThreads),
                     0, st, idx, rows, topk, lens, S, keep, B);
  return hipGetLastError();
}

}  // namespace si
