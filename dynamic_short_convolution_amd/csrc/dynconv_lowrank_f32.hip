// General low-rank kernels instantiated for float storage.
#include "dynconv_lowrank_kernels.hpp"

namespace dynconv {

hipError_t lowrank_dispatch_f32(const LowRankParams& p, const LowRankPlan& pl, int W, bool bwd, hipStream_t s) {
  return lowrank_dispatch<float>(p, pl, W, bwd, s);
}

}  // namespace dynconv
