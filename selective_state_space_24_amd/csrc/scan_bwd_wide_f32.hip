// The backward kernel for one A per head, dstate above 16 and the zero-order hold, f32 io.
#include "scan_bwd_wide.h"

namespace ssm {

hipError_t launch_bwd_wide_f32(const BwdParams& q, hipStream_t stream) {
  return wide_io<float>(q, stream);
}

}  // namespace ssm
