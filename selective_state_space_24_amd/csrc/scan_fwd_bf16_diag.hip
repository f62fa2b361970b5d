// Kernel instantiations for bf16 io, diagonal A per channel.
#include "scan_kernels.h"

namespace ssm {
hipError_t launch_bf16_diag(const ScanParams& p, hipStream_t stream) {
  return launch_n<bf16_bits, false>(p, stream);
}
}  // namespace ssm
