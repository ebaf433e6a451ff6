// GEMM dispatch by mode, form and shape.
#include "gemm_common.hpp"

namespace hq {

hipError_t launch_gemm_direct(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev);

hipError_t launch_gemm(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  return launch_gemm_direct(s, p, dev);
}

}  // namespace hq
