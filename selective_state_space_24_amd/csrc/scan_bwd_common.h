// Helpers shared by the gfx950 backward kernels (scan_bwd.hip, scan_bwd_wide.hip).
#pragma once
#include "scan_kernels.h"

namespace ssm {

// v of lane l plus v of lane l ^ off (the same sum in both lanes): off 16 and 32 by the
// lane-swap instructions, which leave {v(l), v(l ^ off)} in the two results in every lane (no
// LDS round trip); smaller offsets by a permute
__device__ __forceinline__ float xor_sum(float v, int off) {
  const uint32_t u = __float_as_uint(v);
  if (off == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v + __shfl_xor(v, off);
}

// sigmoid(v) from delta = softplus(v): e^delta = 1 + e^v gives sigmoid(v) = 1 - e^-delta. For
// small delta the series delta (1 - delta/2 + delta^2/6 - delta^3/24) avoids the cancellation
// (its first dropped term is below 1e-7 relative at delta = 0.1).
__device__ __forceinline__ float sigmoid_from_softplus(float dl) {
  const float series = dl * fmaf(dl, fmaf(dl, fmaf(dl, -1.0f / 24.0f, 1.0f / 6.0f), -0.5f), 1.0f);
  return dl < 0.1f ? series : 1.0f - __builtin_amdgcn_exp2f(-dl * kLog2e);
}

// two consecutive elements (a, b) at p, which holds a pair: one 4-byte (bf16) or 8-byte store
__device__ __forceinline__ void store_pair(bf16_bits* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}
__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

}  // namespace ssm
