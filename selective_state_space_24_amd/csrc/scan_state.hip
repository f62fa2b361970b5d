// The final state of a scan with no time steps: a copy of the initial state, or zeros. A plain
// kernel rather than a runtime memset or copy, so that callers may capture the call in a graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_internal.h"

namespace ssm {

__global__ void __launch_bounds__(256) state_copy_kernel(const float* __restrict__ src,
                                                         float* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.0f;
}

// The SIMD (0..3 of its CU) of every wavefront of 8-wavefront workgroups, as the scan kernel with
// independent wavefronts is launched: field SIMD_ID (bits 5:4) of the hardware register HW_ID.
// That kernel's pacing assumes wavefronts w and w ^ 4 of a workgroup share a SIMD.
__global__ void __launch_bounds__(512) wave_simd_kernel(int32_t* __restrict__ out) {
  constexpr int kHwRegHwId = 4, kSimdIdOffset = 4, kSimdIdBits = 2;
  if ((threadIdx.x & 63) == 0) {
    const unsigned v = __builtin_amdgcn_s_getreg(kHwRegHwId | (kSimdIdOffset << 6) |
                                                 ((kSimdIdBits - 1) << 11));
    out[(int64_t)blockIdx.x * 8 + (threadIdx.x >> 6)] = (int32_t)v;
  }
}

hipError_t launch_wave_simd(int32_t* out, int32_t nworkgroups, hipStream_t stream) {
  if (nworkgroups <= 0) return hipSuccess;
  hipLaunchKernelGGL(wave_simd_kernel, dim3((unsigned)nworkgroups), dim3(512), 0, stream, out);
  return hipGetLastError();
}

hipError_t launch_state_copy(const float* src, float* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(state_copy_kernel, dim3(grid), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

}  // namespace ssm
