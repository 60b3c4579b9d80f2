// Product-key addressing for Sparse Delta Memory: launch selection.  The
// kernel and its design notes are in score_topk_impl.h; its instances are
// compiled in score_topk_t{1,2,4,8}.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "score_topk_impl.h"

namespace sdm {

extern template hipError_t launch_score_t<1>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_t<2>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_t<4>(const ScoreArgs&, bool, int, hipStream_t);
extern template hipError_t launch_score_t<8>(const ScoreArgs&, bool, int, hipStream_t);

size_t score_topk_lds_bytes(int n_sub, int W, int R) {
  (void)n_sub;
  return score_smem(W, R).total;
}

hipError_t launch_score_topk(const ScoreArgs& a, bool bf16, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int tiles = (a.n_sub + 15) / 16;
  const int nt = (tiles + kWaves - 1) / kWaves;  // sub-key tiles per wave
  const int g = pruned_grid_size(a.W > a.R ? a.W : a.R);
  const int npl2 = (g + 63) / 64;
  if (npl2 > kGridMax / 64) return hipErrorInvalidValue;
  if (nt <= 1) return launch_score_t<1>(a, bf16, npl2, stream);
  if (nt <= 2) return launch_score_t<2>(a, bf16, npl2, stream);
  if (nt <= 4) return launch_score_t<4>(a, bf16, npl2, stream);
  if (nt <= 8) return launch_score_t<8>(a, bf16, npl2, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdm
