// Streaming kernels instantiated for bf16_t storage.
#include "dynconv_stream_kernels.hpp"

namespace dynconv {

hipError_t stream_dispatch_bf16(const StreamParams& p, const StreamPlan& plan, int W, bool is_static, bool bwd,
                              hipStream_t s) {
  return stream_dispatch<bf16_t>(p, plan, W, is_static, bwd, s);
}

}  // namespace dynconv
