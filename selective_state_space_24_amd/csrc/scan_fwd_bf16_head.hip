// Kernel instantiations for bf16 io, one A per head.
#include "scan_kernels.h"

namespace ssm {
hipError_t launch_bf16_head(const ScanParams& p, hipStream_t stream) {
  return launch_n<bf16_bits, true>(p, stream);
}
}  // namespace ssm
