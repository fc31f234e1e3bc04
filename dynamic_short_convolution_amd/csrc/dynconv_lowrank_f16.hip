// General low-rank kernels instantiated for f16_t storage.
#include "dynconv_lowrank_kernels.hpp"

namespace dynconv {

hipError_t lowrank_dispatch_f16(const LowRankParams& p, const LowRankPlan& pl, int W, bool bwd, hipStream_t s) {
  return lowrank_dispatch<f16_t>(p, pl, W, bwd, s);
}

}  // namespace dynconv
