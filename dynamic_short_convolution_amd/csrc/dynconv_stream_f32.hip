// Streaming kernels instantiated for float storage.
#include "dynconv_stream_kernels.hpp"

namespace dynconv {

hipError_t stream_dispatch_f32(const StreamParams& p, const StreamPlan& plan, int W, bool is_static, bool bwd,
                              hipStream_t s) {
  return stream_dispatch<float>(p, plan, W, is_static, bwd, s);
}

}  // namespace dynconv
