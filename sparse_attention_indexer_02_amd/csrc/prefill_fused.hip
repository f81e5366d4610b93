// Prefill score and top-K in one kernel (the score writeback and the
// selection input are costs the DoSA reading notes, section 5, name; here
// the selection reads each score row back while it is still in cache, and
// its VALU and LDS work runs beside other workgroups' MFMA work on the same
// CU instead of in a kernel of its own).
//
// One workgroup owns 4 QPW query rows (the score kernel's grouping, longest
// rows first): it scores them over all their visible keys exactly as
// score_mfma_shared does (score_group_shared, the same bits), writes the
// score rows to the workspace, and then takes each row's top-K with its 256
// threads (topk_row_block with 32 scores per thread, the same algorithm and
// result as the top-K kernel), with the segment-witness merge when asked.
// Shapes: shared bf16 keys that fit one key segment (a 2 MiB key matrix),
// rows of at most 8192 keys, K <= 2048 (idx_score_topk_fused).  Measured on
// MI355X it is slower than the score kernel followed by the top-K kernel:
// while one workgroup selects, its four waves leave the MFMA units of their
// SIMDs to the other resident workgroups, and its selection runs with four
// waves per row instead of eight, so the selection's latency is exposed
// rather than hidden; idx_score_topk therefore keeps the two kernels.
#include "score_shared.hpp"
#include "topk_block.hpp"

namespace si {

constexpr int kFusedThreads = 256;

template <int MT, int KS, int QPW, bool WIT>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(3))) void score_topk_prefill(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int64_t w_stride, const int32_t* __restrict__ vis_len, int n_q, int H, int64_t n_k,
    int64_t max_vis, float* __restrict__ scores, TopkArgs ta) {
  constexpr int QB = 4 * QPW;
  // the score loop's key tiles and the top-K's state never live at once
  __shared__ union alignas(16) {
    unsigned char score[score_lds_bytes<KS>()];
    TopkSmem<kFusedThreads> topk;
  } sm;
  const int G = (n_q + QB - 1) / QB;
  const int g = G - 1 - (int)blockIdx.x;  // longest rows first
  score_group_shared<MT, KS, QPW>(q, k, w, w_stride, vis_len, H, n_k, max_vis, scores, max_vis,
                                  nullptr, n_q, g, 0, max_vis, sm.score);
  // the rows' scores, stored by all four waves, are visible to the whole
  // workgroup past this barrier, and the LDS is free for the top-K
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < QB; ++i) {
    const int r = g * QB + i;
    if (r >= n_q) break;
    topk_row_block<kFusedThreads, kBN / kFusedThreads, WIT, false>(ta, r, 0, sm.topk);
    __syncthreads();  // the next row reuses the LDS
  }
}

bool score_topk_fused_supported(const ScoreArgs& a, int K) {
  if (!score_mfma_supported(a) || a.k_row_offset != nullptr || a.k_dtype != SI_BF16) return false;
  if (a.max_vis > kBN || K > kBK) return false;
  if (a.n_k * a.D * 2 > (int64_t)INT32_MAX) return false;
  int64_t seg_keys;
  return key_segments(a.max_vis < a.n_k ? a.max_vis : a.n_k, a.D, &seg_keys) == 1;
}

hipError_t launch_score_topk_fused(const ScoreArgs& a, const TopkArgs& ta, hipStream_t st) {
  if (a.n_q == 0 || a.max_vis == 0) {  // nothing visible: every row is padding
    return launch_topk(ta, st);
  }
  const int MT = a.H <= 32 ? 1 : 2;
  const int QPW = MT == 1 ? 2 : 1;
  const unsigned grid = (unsigned)((a.n_q + 4 * QPW - 1) / (4 * QPW));
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* k = reinterpret_cast<const uint16_t*>(a.k);
  const bool wit = ta.wit_lens != nullptr;
#define SI_FUSED(MT_, KS_, QPW_, WIT_)                                                           \
  hipLaunchKernelGGL((score_topk_prefill<MT_, KS_, QPW_, WIT_>), dim3(grid), dim3(kFusedThreads), \
                     0, st, q, k, a.w, a.w_row_stride, a.vis_len, a.n_q, a.H, a.n_k, a.max_vis,   \
                     a.scores, ta)
  if (a.D == 128) {
    if (MT == 2) {
      if (wit) SI_FUSED(2, 8, 1, true); else SI_FUSED(2, 8, 1, false);
    } else {
      if (wit) SI_FUSED(1, 8, 2, true); else SI_FUSED(1, 8, 2, false);
    }
  } else {
    if (MT == 2) {
      if (wit) SI_FUSED(2, 4, 1, true); else SI_FUSED(2, 4, 1, false);
    } else {
      if (wit) SI_FUSED(1, 4, 2, true); else SI_FUSED(1, 4, 2, false);
    }
  }
#undef SI_FUSED
  return hipGetLastError();
}

}  // namespace si
