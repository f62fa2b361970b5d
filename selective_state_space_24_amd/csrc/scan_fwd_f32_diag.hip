// Kernel instantiations for fp32 io, diagonal A per channel.
#include "scan_kernels.h"

namespace ssm {
hipError_t launch_f32_diag(const ScanParams& p, hipStream_t stream) {
  return launch_n<float, false>(p, stream);
}
}  // namespace ssm
