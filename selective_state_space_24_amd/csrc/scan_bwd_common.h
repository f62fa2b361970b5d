// Helpers shared by the gfx950 backward kernels (scan_bwd.hip, scan_bwd_wide.hip).
#pragma once
#include "scan_kernels.h"

namespace ssm {

// DPP row-level moves (within each row of 16 lanes)
constexpr int kDppQuadXor1 = 0xb1;       // quad_perm [1, 0, 3, 2]: lane l ^ 1
constexpr int kDppQuadXor2 = 0x4e;       // quad_perm [2, 3, 0, 1]: lane l ^ 2
constexpr int kDppHalfMirror = 0x141;    // lane 7 - l within each 8
constexpr int kDppRowRor8 = 0x128;       // lane (l + 8) % 16: lane l ^ 8
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// v of lane l plus v of lane l ^ off (the same sum in both lanes): off 16 and 32 by the
// lane-swap instructions, which leave {v(l), v(l ^ off)} in the two results in every lane, off 8
// by a row rotation (no LDS round trip); smaller offsets by a permute
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
  if (off == 8) return v + dpp_f32<kDppRowRor8>(v);
  return v + __shfl_xor(v, off);
}

// sigmoid(v) from delta = softplus(v): e^delta = 1 + e^v gives sigmoid(v) = 1 - e^-delta. For
// small delta the series delta (1 - delta/2 + delta^2/6 - delta^3/24) avoids the cancellation
// (its first dropped term is below 1e-7 relative at delta = 0.1).
__device__ __forceinline__ float sigmoid_from_softplus(float dl) {
  const float series = dl * fmaf(dl, fmaf(dl, fmaf(dl, -1.0f / 24.0f, 1.0f / 6.0f), -0.5f), 1.0f);
  return dl < 0.1f ? series : 1.0f - __builtin_amdgcn_exp2f(-dl * kLog2e);
}

// Sums each of M values (M = 2, 4 or 8) over the 64 lanes of a wavefront, in registers: the
// value pairs are split across lane halves (xor 32, then 16, then 8) with the lane-swap
// instructions and a row rotation, each lane keeping one value of each pair and adding its
// partner's copy, until every lane holds one value; a reduction within the remaining 64 / M
// lanes finishes the sum. Afterwards every lane l holds the total of value l / (64 / M). The
// order of the additions is fixed.
template <int M>
__device__ __forceinline__ float lane_sums(const float (&v)[M]) {
  static_assert(M == 2 || M == 4 || M == 8, "2, 4 or 8 values");
  const int lane = (int)__lane_id();
  float w[M / 2];
#pragma unroll
  for (int k = 0; k < M / 2; ++k) {  // xor 32: lanes < 32 keep value k, the others k + M / 2
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]),
                                                    __float_as_uint(v[k + M / 2]), false, false);
    w[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float x;
  if constexpr (M == 2) {
    x = w[0];
  } else {
    float y[M / 4];
#pragma unroll
    for (int k = 0; k < M / 4; ++k) {  // xor 16: rows 0, 2 keep w[k], rows 1, 3 w[k + M / 4]
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[k]),
                                                      __float_as_uint(w[k + M / 4]), false, false);
      y[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (M == 4) {
      x = y[0];
    } else {  // xor 8: lanes with bit 3 clear keep y[0], the others y[1]
      const float s0 = y[0] + dpp_f32<kDppRowRor8>(y[0]);
      const float s1 = y[1] + dpp_f32<kDppRowRor8>(y[1]);
      x = (lane & 8) ? s1 : s0;
    }
  }
  // the 64 / M lanes that hold the same value
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  if constexpr (M <= 4) x += dpp_f32<kDppRowRor8>(x);
  if constexpr (M == 2) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// row[t .. t + kVec) as its raw 16 bytes (cnt elements valid, the rest zero), for unpack16: one
// 16-byte load (read-once hint) when vec_ok and the chunk is whole, else element loads
template <typename IO>
__device__ __forceinline__ u32x4 load_raw16(const IO* __restrict__ row, int64_t t, int cnt,
                                            bool vec_ok) {
  constexpr int V = IoTraits<IO>::kVec;
  if (vec_ok && cnt == V) return load16<true>(row + t);
  uint32_t ws[4];
  if constexpr (V == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = 2 * k < cnt ? (uint32_t)row[t + 2 * k] : 0u;
      const uint32_t hi = 2 * k + 1 < cnt ? (uint32_t)row[t + 2 * k + 1] : 0u;
      ws[k] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) ws[k] = k < cnt ? __float_as_uint(row[t + k]) : 0u;
  }
  return u32x4{ws[0], ws[1], ws[2], ws[3]};
}

// kVec io values as one 16-byte word (bf16 rounded to nearest even, as store_chunk does)
template <typename IO>
__device__ __forceinline__ u32x4 pack16(const float (&v)[IoTraits<IO>::kVec]) {
  uint32_t ws[4];
  if constexpr (IoTraits<IO>::kVec == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) ws[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) ws[k] = __float_as_uint(v[k]);
  }
  return u32x4{ws[0], ws[1], ws[2], ws[3]};
}

// stores a word made by pack16 at row[t ..): whole (write-once hint) when vec_ok and all kVec
// elements are valid, else its first cnt elements one by one
template <typename IO>
__device__ __forceinline__ void store_raw16(IO* __restrict__ row, int64_t t, int cnt, bool vec_ok,
                                            const u32x4 w) {
  constexpr int V = IoTraits<IO>::kVec;
  if (vec_ok && cnt == V) {
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(row + t));
    return;
  }
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < V; ++e) {
    if (e >= cnt) continue;
    if constexpr (V == 8) {
      row[t + e] = (IO)((ws[e / 2] >> (16 * (e & 1))) & 0xffffu);
    } else {
      row[t + e] = __uint_as_float(ws[e]);
    }
  }
}

}  // namespace ssm
