// The backward kernel for one A per head, dstate above 16 and the zero-order hold, bf16 io.
#include "scan_bwd_wide.h"

namespace ssm {

hipError_t launch_bwd_wide_bf16(const BwdParams& q, hipStream_t stream) {
  return wide_io<bf16_bits>(q, stream);
}

}  // namespace ssm
