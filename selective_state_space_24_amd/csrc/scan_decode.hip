// gfx950 kernel of the single-step recurrent update (decoding one token per sequence).
//
// The selective SSM is a recurrence, so generating one token needs only the previous state:
// h <- exp(delta A) h + delta B x and y = C.h + D x (then the gate), with constant work and
// memory per step (page "NL-345", §1 and §2 "Computation", the recurrent mode used for
// autoregressive inference). The state (batch, dim, N) fp32 is read and written once per step,
// so the kernel is bound by HBM bandwidth on it.
//
// Mapping: TPC threads per channel (TPC = N/4 rounded up to a power of two, at most 32), each
// owning 4 consecutive states of one channel for BPT consecutive batch entries. Consecutive
// threads touch consecutive 16-byte pieces of the state of one batch entry; the per-channel
// parameters (A row, D, bias) are loaded once per thread, and the BPT entries' loads are all in
// flight together. The readout sum over the channel's states is reduced over its TPC lanes with
// cross-lane shuffles; lane 0 of the group stores y.
//
// Two versions: decode_vec_kernel, when the state, A and B/C rows allow 4-element vector access,
// first issues every load of its BPT batch entries (addresses clamped into the tensors, so that
// no load is conditional) and only then computes; decode_kernel takes any strides and sizes,
// with guarded loads.
#include "scan_kernels.h"

namespace ssm {

constexpr int kDecodeBatchPerThread = 8;

// 4 consecutive io elements as fp32: one 8- or 16-byte load when `vec`, else guarded loads
template <typename IO>
__device__ __forceinline__ void load4(const IO* __restrict__ p, int64_t stride, int cnt, bool vec,
                                      float (&out)[4]) {
  if (vec) {
    if constexpr (sizeof(IO) == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      out[0] = __uint_as_float(w.x << 16); out[1] = __uint_as_float(w.x & 0xffff0000u);
      out[2] = __uint_as_float(w.y << 16); out[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
      const float4 v = *reinterpret_cast<const float4*>(p);
      out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = k < cnt ? to_f32(p[k * stride]) : 0.0f;
  }
}

// Sum of v over aligned groups of TPC lanes (every lane of a group gets the sum): DPP within
// quads, half rows and rows, a shuffle across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int TPC>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (TPC >= 2) v += dpp_mov<0xb1>(v);   // quad_perm [1, 0, 3, 2]
  if constexpr (TPC >= 4) v += dpp_mov<0x4e>(v);   // quad_perm [2, 3, 0, 1]
  if constexpr (TPC >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror: lane i <-> 7 - i of 8
  if constexpr (TPC >= 16) v += dpp_mov<0x140>(v); // row_mirror: lane i <-> 15 - i of 16
  if constexpr (TPC >= 32) v += __shfl_xor(v, 16);
  return v;
}

// 4 io elements of a 4-aligned position as fp32 (one 8- or 16-byte load)
template <typename IO>
__device__ __forceinline__ void load4v(const IO* __restrict__ p, float (&out)[4]) {
  if constexpr (sizeof(IO) == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    out[0] = __uint_as_float(w.x << 16); out[1] = __uint_as_float(w.x & 0xffff0000u);
    out[2] = __uint_as_float(w.y << 16); out[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
}

template <typename IO, int TPC, bool HEAD, bool GATE>
__global__ void __launch_bounds__(256) decode_vec_kernel(const ScanParams p) {
  constexpr int BPT = kDecodeBatchPerThread;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t d_raw = gid / TPC;
  const int sub = (int)(gid % TPC);
  const bool dlive = d_raw < p.dim;
  const int64_t d = dlive ? d_raw : p.dim - 1;  // clamped: every load stays in the tensors
  const int64_t dr = HEAD ? d / p.headdim : d;
  const int64_t g = d / (p.dim / p.ngroups);
  const bool nlive = sub * 4 < p.N;
  const int n0 = nlive ? sub * 4 : 0;
  const int64_t b0 = (int64_t)blockIdx.y * BPT;

  float a[4];
  if constexpr (HEAD) {
    const float ah = p.A[dr] * kLog2e;
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = ah;
  } else {
    load4v<float>(p.A + d * p.N + n0, a);
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] *= kLog2e;
  }
  const float Dd = p.D ? p.D[d] : 0.0f;
  const float bias = p.delta_bias ? p.delta_bias[dr] : 0.0f;

  const IO* X = static_cast<const IO*>(p.x);
  const IO* DL = static_cast<const IO*>(p.delta);
  const IO* Bm = static_cast<const IO*>(p.B);
  const IO* Cm = static_cast<const IO*>(p.C);
  const IO* Z = static_cast<const IO*>(p.z);
  IO* Y = static_cast<IO*>(p.y);

  // every load of the BPT entries first
  float h[BPT][4], bv[BPT][4], cv[BPT][4], xv[BPT], dv[BPT], zv[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int64_t b = min(b0 + i, p.batch - 1);
    load4v<float>(p.h0 + (b * p.dim + d) * p.N + n0, h[i]);
    load4v<IO>(Bm + b * p.B_sb + g * p.B_sg + n0, bv[i]);
    load4v<IO>(Cm + b * p.C_sb + g * p.C_sg + n0, cv[i]);
    xv[i] = to_f32(X[b * p.x_sb + d * p.x_sd]);
    dv[i] = to_f32(DL[b * p.dl_sb + dr * p.dl_sd]);
    zv[i] = GATE ? to_f32(Z[b * p.z_sb + d * p.z_sd]) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const bool blive = b0 + i < p.batch;
    const float v = dv[i] + bias;
    const float dl = p.softplus ? softplus_f32(v) : v;
    const float u = dl * xv[i];
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h[i][k] = fmaf(__builtin_amdgcn_exp2f(dl * a[k]), h[i][k], u * bv[i][k]);
      part = fmaf(cv[i][k], h[i][k], part);
    }
    if (dlive && nlive && blive)
      *reinterpret_cast<float4*>(p.hfin + ((b0 + i) * p.dim + d) * p.N + n0) =
          make_float4(h[i][0], h[i][1], h[i][2], h[i][3]);
    part = group_sum<TPC>(nlive ? part : 0.0f);
    if (dlive && blive && sub == 0) {
      float y = fmaf(Dd, xv[i], part);
      if constexpr (GATE) y *= silu_f32(zv[i]);
      store_elem(Y + (b0 + i) * p.y_sb + d * p.y_sd, y);
    }
  }
}

template <typename IO, int TPC, bool HEAD, bool GATE>
__global__ void __launch_bounds__(256) decode_kernel(const ScanParams p) {
  constexpr int BPT = kDecodeBatchPerThread;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t d_raw = gid / TPC;
  const int sub = (int)(gid % TPC);
  const bool dlive = d_raw < p.dim;
  const int64_t d = dlive ? d_raw : 0;
  const int64_t dr = HEAD ? d / p.headdim : d;
  const int64_t g = d / (p.dim / p.ngroups);
  const int n0 = sub * 4;
  const int cnt = (int)min<int64_t>(4, max<int64_t>(0, p.N - n0));
  const bool full = cnt == 4;

  // per-channel parameters, loaded once (with log2 e folded into A)
  float a[4];
  if constexpr (HEAD) {
    const float ah = dlive ? p.A[dr] * kLog2e : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = ah;
  } else {
    if (dlive) load4<float>(p.A + d * p.N + n0, 1, cnt, full && p.a_vec, a);
    else a[0] = a[1] = a[2] = a[3] = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] *= kLog2e;
  }
  const float Dd = (dlive && p.D) ? p.D[d] : 0.0f;
  const float bias = (dlive && p.delta_bias) ? p.delta_bias[dr] : 0.0f;

  const IO* X = static_cast<const IO*>(p.x);
  const IO* DL = static_cast<const IO*>(p.delta);
  const IO* Bm = static_cast<const IO*>(p.B);
  const IO* Cm = static_cast<const IO*>(p.C);
  const IO* Z = static_cast<const IO*>(p.z);
  IO* Y = static_cast<IO*>(p.y);
  const bool svec = p.state_vec != 0 && full;
  const bool bvec = p.bc_vec != 0 && full;

#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int64_t b_raw = (int64_t)blockIdx.y * BPT + i;
    const bool live = dlive && b_raw < p.batch;
    const int64_t b = live ? b_raw : 0;
    float part = 0.0f, xv = 0.0f, zv = 0.0f;
    if (live) {
      xv = to_f32(X[b * p.x_sb + d * p.x_sd]);
      const float v = to_f32(DL[b * p.dl_sb + dr * p.dl_sd]) + bias;
      if constexpr (GATE) zv = to_f32(Z[b * p.z_sb + d * p.z_sd]);
      const float dl = p.softplus ? softplus_f32(v) : v;
      const float u = dl * xv;
      const int64_t so = (b * p.dim + d) * p.N + n0;
      float h[4], bv[4], cv[4];
      load4<float>(p.h0 + so, 1, cnt, svec, h);
      load4<IO>(Bm + b * p.B_sb + g * p.B_sg + n0 * p.B_sn, p.B_sn, cnt, bvec, bv);
      load4<IO>(Cm + b * p.C_sb + g * p.C_sg + n0 * p.C_sn, p.C_sn, cnt, bvec, cv);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = fmaf(__builtin_amdgcn_exp2f(dl * a[k]), h[k], u * bv[k]);
        part = fmaf(cv[k], h[k], part);
      }
      float* st = p.hfin + so;
      if (svec) {
        *reinterpret_cast<float4*>(st) = make_float4(h[0], h[1], h[2], h[3]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k < cnt) st[k] = h[k];
      }
    }
    // sum over the channel's TPC lanes (every lane takes part, live or not)
#pragma unroll
    for (int off = TPC / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, TPC);
    if (live && sub == 0) {
      float y = fmaf(Dd, xv, part);
      if constexpr (GATE) y *= silu_f32(zv);
      store_elem(Y + b * p.y_sb + d * p.y_sd, y);
    }
  }
}

template <typename IO, int TPC, bool HEAD>
static hipError_t decode_launch(const ScanParams& p, hipStream_t stream) {
  const int64_t threads = p.dim * TPC;
  const dim3 grid((unsigned)((threads + 255) / 256),
                  (unsigned)((p.batch + kDecodeBatchPerThread - 1) / kDecodeBatchPerThread));
  const bool vec = p.state_vec && p.bc_vec && (HEAD || p.a_vec);
  if (vec) {
    if (p.z)
      hipLaunchKernelGGL((decode_vec_kernel<IO, TPC, HEAD, true>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_vec_kernel<IO, TPC, HEAD, false>), grid, dim3(256), 0, stream, p);
  } else if (p.z) {
    hipLaunchKernelGGL((decode_kernel<IO, TPC, HEAD, true>), grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_kernel<IO, TPC, HEAD, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename IO, bool HEAD>
static hipError_t decode_n(const ScanParams& p, hipStream_t stream) {
  const int64_t N = p.N;
  if (N <= 4) return decode_launch<IO, 1, HEAD>(p, stream);
  if (N <= 8) return decode_launch<IO, 2, HEAD>(p, stream);
  if (N <= 16) return decode_launch<IO, 4, HEAD>(p, stream);
  if (N <= 32) return decode_launch<IO, 8, HEAD>(p, stream);
  if (N <= 64) return decode_launch<IO, 16, HEAD>(p, stream);
  return decode_launch<IO, 32, HEAD>(p, stream);  // N <= 128 (checked by the caller)
}

hipError_t launch_decode(const ScanParams& p, bool bf16, bool head, hipStream_t stream) {
  if (bf16) return head ? decode_n<bf16_bits, true>(p, stream) : decode_n<bf16_bits, false>(p, stream);
  return head ? decode_n<float, true>(p, stream) : decode_n<float, false>(p, stream);
}

}  // namespace ssm
