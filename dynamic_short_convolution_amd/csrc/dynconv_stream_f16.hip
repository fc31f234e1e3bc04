// Streaming kernels instantiated for f16_t storage.
#include "dynconv_stream_kernels.hpp"

namespace dynconv {

hipError_t stream_dispatch_f16(const StreamParams& p, const StreamPlan& plan, int W, bool is_static, bool bwd,
                              hipStream_t s) {
  return stream_dispatch<f16_t>(p, plan, W, is_static, bwd, s);
}

}  // namespace dynconv
