// Instances of the product-key addressing kernel with 4 stage-1 score(s) per lane.
#include "score_topk_impl.h"

namespace sdm {
template hipError_t launch_score_n<4>(const ScoreArgs&, bool, int, hipStream_t);
}  // namespace sdm
