// Instances of the product-key addressing kernel with 8 sub-key tile(s) per wave.
#include "score_topk_impl.h"

namespace sdm {
template hipError_t launch_score_t<8>(const ScoreArgs&, bool, int, hipStream_t);
}  // namespace sdm
