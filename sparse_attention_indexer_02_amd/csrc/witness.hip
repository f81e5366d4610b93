// Segment-witness merge, in place ("Segment Witnesses" page: Object,
// Implementation rule and contracts).
//
// One wave per row.  Lanes stream the row with 16-byte loads and OR each
// entry's segment bit into a 64-bit occupancy mask; the mask is OR-reduced
// across the wave; lane s (< S_eff) then owns segment s: if it is empty its
// witness e_s = ceil(s L / S_eff) takes slot keep + (number of empty segments
// below s), when that rank is < B.  Only those <= B slots are written.
//
// The segment of an in-range entry, floor(x S_eff / L), comes from an fp32
// quotient estimate corrected once each way with exact 64-bit integer
// arithmetic (the estimate is within 1 of the true floor: the quotient is
// below 64 and the relative error of the estimate is a few 2^-24).
#include "si_internal.hpp"

namespace si {

constexpr int kWitThreads = 256;

__device__ __forceinline__ uint64_t seg_bit(int32_t x, uint32_t L, uint32_t S, uint32_t Se,
                                            float rcpL) {
  if (x < 0) return 0ull;  // padding marks no segment
  uint32_t ux = (uint32_t)x;
  uint32_t seg;
  if (ux >= L) {
    // min(floor(x S_eff / L), S - 1): S - 1 when S_eff == S, else x itself
    // (S_eff == L), clamped.
    seg = (Se == S) ? S - 1 : (ux < S - 1 ? ux : S - 1);
  } else {
    uint64_t num = (uint64_t)ux * Se;
    uint32_t est = (uint32_t)((float)num * rcpL);
    int64_t rem = (int64_t)num - (int64_t)est * (int64_t)L;
    if (rem < 0) --est;
    else if (rem >= (int64_t)L) ++est;
    seg = est;
  }
  return 1ull << seg;
}

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
  if (vec) {
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
  uint32_t lo = (uint32_t)occ, hi = (uint32_t)(occ >> 32);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo |= (uint32_t)__shfl_xor((int)lo, o, 64);
    hi |= (uint32_t)__shfl_xor((int)hi, o, 64);
  }
  occ = ((uint64_t)hi << 32) | lo;

  const bool empty = (uint32_t)lane < Se && !((occ >> lane) & 1ull);
  const uint64_t emask = __ballot(empty);
  if (empty) {
    const int rank = __popcll(emask & ((1ull << lane) - 1ull));
    if (rank < B) {
      const uint64_t e = ((uint64_t)lane * L + Se - 1) / Se;  // ceil(s L / S_eff)
      row[keep + rank] = (int32_t)e;
    }
  }
}

hipError_t launch_witness(int32_t* idx, int32_t rows, int32_t topk, const int32_t* lens,
                          int32_t S, int32_t keep, int32_t B, hipStream_t st) {
  const int per = kWitThreads / 64;
  hipLaunchKernelGGL(witness_merge, dim3((unsigned)((rows + per - 1) / per)), dim3(kWitThreads),
                     0, st, idx, rows, topk, lens, S, keep, B);
  return hipGetLastError();
}

}  // namespace si
