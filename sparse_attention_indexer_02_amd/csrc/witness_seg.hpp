// Segment of a row entry for the segment-witness merge ("Segment
// Witnesses" page: Object, Implementation rule and contracts), shared by the
// merge kernel and the block top-K's fused merge.
//
// The segment of an in-range entry, floor(x S_eff / L), comes from an fp32
// quotient estimate corrected once each way with exact integer arithmetic
// (the estimate is within 1 of the true floor: the quotient is below 64 and
// the relative error of the estimate is a few 2^-24); rows with L < 2^26
// do it in 32 bits, longer ones in 64.
#pragma once

#include "si_internal.hpp"

namespace si {

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

// The same segment for rows with L < 2^26, where x * S_eff < 2^32: the
// product, the estimate's back-multiplication and the remainder all fit 32
// bits (est * L <= num + L < 2^32), so the correction needs no 64-bit math.
__device__ __forceinline__ uint64_t seg_bit32(int32_t x, uint32_t L, uint32_t S, uint32_t Se,
                                              float rcpL) {
  const uint32_t ux = (uint32_t)x;
  uint32_t seg;
  if (ux >= L) {
    seg = (Se == S) ? S - 1 : (ux < S - 1 ? ux : S - 1);
  } else {
    const uint32_t num = ux * Se;
    uint32_t est = (uint32_t)((float)num * rcpL);
    const int32_t rem = (int32_t)(num - est * L);
    est = rem < 0 ? est - 1 : (rem >= (int32_t)L ? est + 1 : est);
    seg = est;
  }
  return x < 0 ? 0ull : 1ull << seg;
}

// Witness e_s = ceil(s L / S_eff) of each segment s < S_eff that occ leaves
// empty, written in ascending s to row[keep + rank] for rank < B; lane s of
// the calling wave owns segment s (every lane of the wave calls it).
__device__ __forceinline__ void write_witnesses(int32_t* row, uint64_t occ, uint32_t L,
                                                uint32_t Se, int keep, int B) {
  // the lane id from the lane masks, so no copy of it computed earlier has
  // to stay live until here (the fused top-K otherwise spills one)
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
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

}  // namespace si
