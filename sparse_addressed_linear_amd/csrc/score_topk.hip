// Product-key addressing for Sparse Delta Memory, for gfx950.
//
// Method ("Sparse Delta Memory", gist.science summaries of paper 2607.07386;
// Spanish page "Mecanismo Central" item 2, French page "Mecanisme Central"):
// the projected key (query) is cut into two halves; each half is scored
// against its own table of n_sub sub-keys (product-key memory); slot
// s = i*n_sub + j scores s1[i] + s2[j]; the top-W (top-R) slots are found
// through topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)) without forming the
// N = n_sub^2 scores.  Weights: softmax over the selected sums.  Order: score
// descending, ties to the lower index (sub-key index in stage 1, slot in
// stage 2).
//
// One workgroup handles kTT tokens of one (b,h) stream:
//   1. half scores for the tile: bf16 -> MFMA v_mfma_f32_16x16x32_bf16
//      (sub-keys x tokens, fp32 accumulate), fp32 -> plain VALU dot products
//      in the same sequential order as a scalar loop; results to LDS.
//   2. stage 1, one wave per (token, half): exact top-m selection.
//   3. stage 2, one wave per token: top-k of the outer sums over the pruned
//      rank grid {(a,b): (a+1)(b+1) <= k} -- a pair outside it is beaten by at
//      least k pairs of its dominating rectangle.  With ties in the fp32 sums
//      that argument can fail, so the best pair just outside the grid is
//      checked and, if it could compete, the full m x m grid is ranked.
// Exact selection of the k best of n values held by one wave: every value
// becomes a unique 64-bit key (order-preserving score bits, then the
// complemented index), a threshold t with k <= #{key >= t} <= cap is found by
// counting with ballots (first guess from the score distribution, then integer
// bisection on keys, which always terminates because keys are unique), the
// keys >= t are compacted to LDS and sorted by a register bitonic network.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "score_topk_impl.h"

namespace sdm {

extern template hipError_t launch_score_n<1>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_n<2>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_n<4>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_n<8>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_n<16>(const ScoreArgs&, bool, int, hipStream_t);

size_t score_topk_lds_bytes(int n_sub, int W, int R) {
  return score_smem(n_sub, W > R ? W : R).total;
}

hipError_t launch_score_topk(const ScoreArgs& a, bool bf16, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int npl = (a.n_sub + 63) / 64;
  const int g = pruned_grid_size(a.W > a.R ? a.W : a.R);
  const int npl2 = (g + 63) / 64;
  if (npl2 > kGridMax / 64) return hipErrorInvalidValue;
  if (npl <= 1) return launch_score_n<1>(a, bf16, npl2, stream);
  if (npl <= 2) return launch_score_n<2>(a, bf16, npl2, stream);
  if (npl <= 4) return launch_score_n<4>(a, bf16, npl2, stream);
  if (npl <= 8) return launch_score_n<8>(a, bf16, npl2, stream);
  if (npl <= 16) return launch_score_n<16>(a, bf16, npl2, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdm
