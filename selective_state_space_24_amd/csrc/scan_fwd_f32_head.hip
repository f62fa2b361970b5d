// Kernel instantiations for fp32 io, one A per head.
#include "scan_kernels.h"

namespace ssm {
hipError_t launch_f32_head(const ScanParams& p, hipStream_t stream) {
  return launch_n<float, true>(p, stream);
}
}  // namespace ssm
