// General low-rank kernels instantiated for bf16_t storage.
#include "dynconv_lowrank_kernels.hpp"

namespace dynconv {

hipError_t lowrank_dispatch_bf16(const LowRankParams& p, const LowRankPlan& pl, int W, bool bwd, hipStream_t s) {
  return lowrank_dispatch<bf16_t>(p, pl, W, bwd, s);
}

}  // namespace dynconv
