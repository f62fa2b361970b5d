// gfx950 forward scan with a complex diagonal A (the a_mode SSM_A_COMPLEX of ssm_scan.h).
//
// The memo page's Figure 10 caption compares SSM parameterisations and stresses complex-valued
// parameters; the recurrence is that of page "NL-345", §2 eq. (2), over complex numbers:
//   Abar_tn = e^(delta_t A_n),  h_tn = Abar_tn h_(t-1)n + delta_t B_tn x_t,
//   y_t = (Re(sum_n C_tn h_tn) + D x_t) silu(z_t),
// with A_n, B_tn, C_tn and h complex and delta, x, z real. e^(delta A) = 2^(delta Re(A) log2 e)
// (cos + i sin)(delta Im(A)); the angle is formed in revolutions, delta Im(A) / 2 pi, and goes to
// the hardware sine and cosine, which take revolutions.
//
// Work split: one workgroup = one wavefront. A channel's NS complex states are spread over LPC
// adjacent lanes, SPL states each, so a wavefront scans 64 / LPC channels of one batch entry;
// each lane's partial Re(C h) is summed over its LPC lanes with DPP adds every step. Splitting
// the states (rather than giving a lane a whole channel) multiplies the number of wavefronts by
// LPC: a Mamba-size layer with a lane per channel fills a fifth of the SIMDs.
//
// Per 16-step tile, the channels' delta (activated), x and z wait in LDS slots, one 16-byte slot
// per (channel, step), where Re(C h) then collects; the tile's B and C values are staged as one
// 16-byte (Re B, Im B, Re C, Im C) entry per (step, state). The next tile's 16-byte global loads
// are issued before the current tile's steps and land in registers meanwhile. D x and the gate
// are applied when the tile's y is written, once per (channel, step) instead of in every lane of
// the channel.
#include "scan_bwd_common.h"

namespace ssm {
namespace {

constexpr int kCT = 16;  // steps per tile
constexpr int kDppRowMirror = 0x140;  // lane 15 - l within each 16

// The sum of v over each aligned group of G lanes (G = 1, 2, 4, 8 or 16), in every lane of the
// group: xor 1 and xor 2 make quad sums, then the mirrors pair each lane with one in the other
// quad (half-row) or the other half-row (row).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<kDppQuadXor1>(v);
  if constexpr (G >= 4) v += dpp_f32<kDppQuadXor2>(v);
  if constexpr (G >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f32<kDppRowMirror>(v);
  return v;
}

template <typename IO, int SPL, int LPC, bool GATE>
__global__ void __launch_bounds__(64) scan_complex_kernel(const ScanParams p) {
  constexpr int NS = SPL * LPC;   // states per channel, padded
  constexpr int CPW = 64 / LPC;   // channels per wavefront
  constexpr int V = IoTraits<IO>::kVec;
  constexpr int CH = kCT / V;     // 16-byte pieces per row of a tile
  constexpr int kSlot = kCT + 1;  // slots per channel (odd in 16-byte units: no bank conflicts)
  constexpr int BC_ITEMS = 4 * NS * CH, BC_PER = (BC_ITEMS + 63) / 64;
  constexpr int IN_ITEMS = CPW * CH, IN_PER = (IN_ITEMS + 63) / 64;
  // [t][n]: (Re B, Im B, Re C, Im C)
  __shared__ __align__(16) f32x4 s_bc[kCT * NS];
  // [channel][t]: (delta, x, z, Re(C h))
  __shared__ __align__(16) f32x4 s_in[CPW * kSlot];

  const int lane = threadIdx.x;
  const int ch = lane / LPC, q = lane % LPC;
  const int64_t blk_per_b = (p.dim + CPW - 1) / CPW;
  const int64_t b = blockIdx.x / blk_per_b;
  const int64_t d0 = (blockIdx.x % blk_per_b) * CPW;
  const int64_t grp = d0 / (p.dim / p.ngroups);
  const int64_t L = p.L, N = p.N;
  const bool vec = p.vec_io != 0, bc_vec = p.bc_vec != 0;

  // this lane's states n = q SPL + j: A_n as Re(A) log2 e for exp2 and Im(A) / 2 pi for the
  // rotation in revolutions; padding states (n >= N) and channels (d >= dim) have A = 0 and
  // B = 0 and stay at zero
  constexpr float kInv2Pi = 0.15915494309189535f;
  const int64_t d = d0 + ch;
  const bool live = d < p.dim;
  float ar[SPL], ai[SPL], hr[SPL], hi[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int64_t n = q * SPL + j;
    const bool on = live && n < N;
    ar[j] = on ? p.A[(d * N + n) * 2] * kLog2e : 0.0f;
    ai[j] = on ? p.A[(d * N + n) * 2 + 1] * kInv2Pi : 0.0f;
    hr[j] = 0.0f;
    hi[j] = 0.0f;
  }
  f32x4* const slot = s_in + ch * kSlot;

  // The items of a tile: B/C item i is a 16-byte piece c of row (part, n), part fastest across
  // lanes so that the LDS writes of a piece's steps fall in consecutive words; input item i is
  // piece c of channel row r. Pieces that are whole and aligned are loaded ahead as raw words.
  const IO* const Bg = static_cast<const IO*>(p.B) + b * p.B_sb + grp * p.B_sg;
  const IO* const Cg = static_cast<const IO*>(p.C) + b * p.C_sb + grp * p.C_sg;
  auto bc_src = [&](int i) {
    const int part = i % 4, n = (i / 4) % NS;
    return (part < 2 ? Bg : Cg) +
           ((part & 1) * N + (n < N ? n : 0)) * (part < 2 ? p.B_sn : p.C_sn);
  };
  auto bc_cnt = [&](int i, int len) {
    const int n = (i / 4) % NS, c = i / (4 * NS);
    return n < N ? max(0, min(V, len - c * V)) : 0;
  };
  auto in_row = [&](int i) {
    const int64_t dr = d0 + i / CH;
    return dr < p.dim ? dr : int64_t(-1);
  };
  auto in_cnt = [&](int i, int len) {
    return in_row(i) >= 0 ? max(0, min(V, len - (i % CH) * V)) : 0;
  };
  const IO* const xb = static_cast<const IO*>(p.x) + b * p.x_sb;
  const IO* const db = static_cast<const IO*>(p.delta) + b * p.dl_sb;
  const IO* const zb = GATE ? static_cast<const IO*>(p.z) + b * p.z_sb : nullptr;

  u32x4 wbc[BC_PER], wx[IN_PER], wd[IN_PER], wz[IN_PER];
  auto issue = [&](int64_t t0) {
    const int len = (int)min<int64_t>(kCT, L - t0);
#pragma unroll
    for (int k = 0; k < BC_PER; ++k) {
      const int i = k * 64 + lane;
      if ((BC_ITEMS % 64 == 0 || i < BC_ITEMS) && bc_vec && bc_cnt(i, len) == V)
        wbc[k] = load16<false>(bc_src(i) + t0 + (i / (4 * NS)) * V);
    }
#pragma unroll
    for (int k = 0; k < IN_PER; ++k) {
      const int i = k * 64 + lane;
      if ((IN_ITEMS % 64 == 0 || i < IN_ITEMS) && vec && in_cnt(i, len) == V) {
        const int64_t r = in_row(i), t = t0 + (i % CH) * V;
        wx[k] = load16<true>(xb + r * p.x_sd + t);
        wd[k] = load16<true>(db + r * p.dl_sd + t);
        if constexpr (GATE) wz[k] = load16<true>(zb + r * p.z_sd + t);
      }
    }
  };
  // the tile's pieces into LDS: the loaded words, else element loads (ragged or unaligned
  // pieces); padding steps, states and channels are zero
  auto commit = [&](int64_t t0) {
    const int len = (int)min<int64_t>(kCT, L - t0);
#pragma unroll
    for (int k = 0; k < BC_PER; ++k) {
      const int i = k * 64 + lane;
      if (BC_ITEMS % 64 == 0 || i < BC_ITEMS) {
        const int part = i % 4, n = (i / 4) % NS, c = i / (4 * NS);
        const int cnt = bc_cnt(i, len);
        float v[V];
        if (bc_vec && cnt == V) unpack16<IO>(wbc[k], v);
        else load_chunk<IO, false>(bc_src(i), t0 + c * V, cnt, false, v);
        float* dst = reinterpret_cast<float*>(s_bc) + (c * V * NS + n) * 4 + part;
#pragma unroll
        for (int e = 0; e < V; ++e) dst[e * NS * 4] = v[e];
      }
    }
#pragma unroll
    for (int k = 0; k < IN_PER; ++k) {
      const int i = k * 64 + lane;
      if (IN_ITEMS % 64 == 0 || i < IN_ITEMS) {
        const int64_t r = in_row(i);
        const int c = i % CH, cnt = in_cnt(i, len);
        float tx[V], td[V], tz[V];
        if (vec && cnt == V) {
          unpack16<IO>(wx[k], tx);
          unpack16<IO>(wd[k], td);
          if constexpr (GATE) unpack16<IO>(wz[k], tz);
        } else {
          const int64_t rr = r >= 0 ? r : 0;
          load_chunk<IO, true>(xb + rr * p.x_sd, t0 + c * V, cnt, false, tx);
          load_chunk<IO, true>(db + rr * p.dl_sd, t0 + c * V, cnt, false, td);
          if constexpr (GATE) load_chunk<IO, true>(zb + rr * p.z_sd, t0 + c * V, cnt, false, tz);
        }
        const float bias = (r >= 0 && p.delta_bias) ? p.delta_bias[r] : 0.0f;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float v = td[e] + bias;
          const float dl = e < cnt ? (p.softplus ? softplus_f32(v) : v) : 0.0f;
          s_in[(i / CH) * kSlot + c * V + e] = f32x4{dl, tx[e], GATE ? tz[e] : 0.0f, 0.0f};
        }
      }
    }
  };

  if (L > 0) issue(0);
  for (int64_t t0 = 0; t0 < L; t0 += kCT) {
    const int len = (int)min<int64_t>(kCT, L - t0);
    __syncthreads();  // the previous tile's y phase is done with the slots
    commit(t0);
    if (t0 + kCT < L) issue(t0 + kCT);
    __syncthreads();

#pragma unroll 4
    for (int t = 0; t < kCT; ++t) {
      const float2 in = *reinterpret_cast<const float2*>(&slot[t]);
      const float dl = in.x;
      const float u = dl * in.y;
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const f32x4 bc = s_bc[t * NS + q * SPL + j];
        const float mag = __builtin_amdgcn_exp2f(dl * ar[j]);
        // the angle's whole turns dropped: the hardware sine and cosine take a bounded range
        const float rev = __builtin_amdgcn_fractf(dl * ai[j]);
        const float dr = mag * __builtin_amdgcn_cosf(rev);
        const float di = mag * __builtin_amdgcn_sinf(rev);
        // h <- Abar h + delta B x
        const float nr = fmaf(dr, hr[j], fmaf(-di, hi[j], u * bc.x));
        const float ni = fmaf(dr, hi[j], fmaf(di, hr[j], u * bc.y));
        hr[j] = nr;
        hi[j] = ni;
        // Re(C h)
        acc = fmaf(bc.z, nr, fmaf(-bc.w, ni, acc));
      }
      acc = group_sum<LPC>(acc);
      if (q == 0) slot[t].w = acc;
    }
    __syncthreads();
    // y = (Re(C h) + D x) silu(z) for the tile's valid steps, one 16-byte piece of a row per item
#pragma unroll
    for (int k = 0; k < IN_PER; ++k) {
      const int i = k * 64 + lane;
      if (IN_ITEMS % 64 == 0 || i < IN_ITEMS) {
        const int64_t r = in_row(i);
        const int c = i % CH, cnt = in_cnt(i, len);
        if (cnt > 0) {
          const float Dd = p.D ? p.D[r] : 0.0f;
          float o[V];
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const f32x4 sl = s_in[(i / CH) * kSlot + c * V + e];
            float yy = fmaf(Dd, sl.y, sl.w);
            if constexpr (GATE) yy *= silu_f32(sl.z);
            o[e] = yy;
          }
          store_chunk<IO>(static_cast<IO*>(p.y) + b * p.y_sb + r * p.y_sd, t0 + c * V, cnt,
                          vec && cnt == V, o);
        }
      }
    }
  }
}

template <typename IO, int SPL, int LPC>
hipError_t launch_split(const ScanParams& p, hipStream_t stream) {
  constexpr int CPW = 64 / LPC;
  const dim3 grid((unsigned)(p.batch * ((p.dim + CPW - 1) / CPW))), block(64);
  if (p.z)
    hipLaunchKernelGGL((scan_complex_kernel<IO, SPL, LPC, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((scan_complex_kernel<IO, SPL, LPC, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// states per lane x lanes per channel, by the padded state count: the fastest of the splits
// measured on a Mamba-130M-size layer (batch 8, 1536 channels, L 2048, bf16)
template <typename IO>
hipError_t launch_io(const ScanParams& p, hipStream_t stream) {
  if (p.N <= 4) return launch_split<IO, 1, 4>(p, stream);
  if (p.N <= 8) return launch_split<IO, 2, 4>(p, stream);
  if (p.N <= 16) return launch_split<IO, 2, 8>(p, stream);
  return launch_split<IO, 4, 8>(p, stream);  // N <= 32 (checked by the caller)
}

}  // namespace

hipError_t launch_complex(const ScanParams& p, bool bf16, hipStream_t stream) {
  if (p.batch == 0 || p.L == 0) return hipSuccess;
  return bf16 ? launch_io<bf16_bits>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace ssm
