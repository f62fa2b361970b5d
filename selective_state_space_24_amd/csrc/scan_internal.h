// Internal launch parameters shared by the host dispatch and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Channels handled by one workgroup: one channel per lane of a 64-wide wavefront.
constexpr int kChannelsPerGroup = 64;
// Wavefronts per workgroup; they split the states of the workgroup's channels.
constexpr int kWavesPerGroup = 4;
constexpr int kTB = 32;       // time steps per compute tile
constexpr int kLT = 2 * kTB;  // time steps per load tile (128 bytes of bf16 per row); segments
                              // along L start at multiples of it
constexpr int kCkptStep = 8;  // steps between the states the backward checkpoint pass stores

struct ScanParams {
  // inputs / outputs (device pointers); element type is the io dtype unless noted
  const void* x;
  const void* delta;
  const float* A;           // (dim, N) or (nheads,)
  const void* B;
  const void* C;
  const float* D;           // nullable
  const void* z;            // nullable
  const float* delta_bias;  // nullable
  void* y;
  const float* h0;          // nullable: initial state (batch, dim, N) fp32
  float* hfin;              // nullable: final state (batch, dim, N) fp32
  float* ckpt;              // backward checkpoints: the state before every kCkptStep-th step,
                            // ckpt[((b * ntiles + k) * N + n) * dim + d] (channel-contiguous)
  int64_t ntiles;           // ceil(L / kCkptStep), the number of checkpoints per channel
  // per-segment summaries for sequences split along L (nullable when nseg == 1):
  // hend[((b * dim + d) * nseg + s) * N + n] and dsum[(b * dim + d) * nseg + s]
  float* hend;
  float* dsum;

  int64_t batch, dim, L, N, ngroups, headdim;
  int64_t x_sb, x_sd, dl_sb, dl_sd, B_sb, B_sg, B_sn, C_sb, C_sg, C_sn, z_sb, z_sd, y_sb, y_sd;

  int64_t groups_per_batch;  // ceil(dim / 64)
  int64_t seg_len;           // time steps per segment (multiple of the time tile)
  int32_t nseg;              // segments along L
  int32_t softplus;          // apply softplus to delta + bias
  int32_t vec_io;            // x/delta/z/y rows allow 16-byte vector access
  int32_t bc_vec;            // B/C rows allow 16-byte vector access
  int32_t zoh;               // zero-order-hold B discretisation instead of delta * B
  int32_t state_vec;         // decode: the state allows 16-byte access (N % 4 == 0, aligned)
  int32_t a_vec;             // decode: rows of A allow 16-byte access
  int32_t four_wave;         // bf16 io, 8 < N <= 16: run scan_fwd_kernel rather than the kernel
                             // with independent wavefronts (chosen by the segment planner)
};

// One launcher per (io dtype, A mode); each is compiled in its own translation unit.
hipError_t launch_bf16_diag(const ScanParams& p, hipStream_t stream);
hipError_t launch_bf16_head(const ScanParams& p, hipStream_t stream);
hipError_t launch_f32_diag(const ScanParams& p, hipStream_t stream);
hipError_t launch_f32_head(const ScanParams& p, hipStream_t stream);
// one recurrent step per sequence: reads the state at h0, writes it at hfin (may be equal)
hipError_t launch_decode(const ScanParams& p, bool bf16, bool head, hipStream_t stream);
// Arguments of the backward pass: the forward's (f, single segment) and the gradients. dy has
// the strides of y, dx those of x, ddelta those of delta, dz those of z; dB, dC are fp32 with
// the strides of B and C. The *_part arrays are workspace partials reduced by the last kernels.
struct BwdParams {
  ScanParams f;
  const void* dy;
  void* dx;
  void* ddelta;
  void* dz;       // nullable (no gate)
  float* dA;      // (dim, N)
  float* dB;
  float* dC;
  float* dD;      // nullable
  float* dbias;   // nullable
  float* dh0;     // nullable
  float* dB_part; // (batch, groups_per_batch, N, L)
  float* dC_part;
  float* dA_part; // (batch, dim, N)
  float* dD_part; // (batch, dim)
  float* dbias_part;
  int32_t pair_out;  // dx, ddelta, dz allow stores of two consecutive elements (aligned to 2
                     // elements, with the strides of x, delta, z)
};
hipError_t launch_bwd(const BwdParams& q, bool bf16, hipStream_t stream);
// Chunked matrix form of the head-mode forward pass (bf16 io, MFMA). ssd_supported checks the
// shape and access conditions it needs (dstate 64 or 128, 64-channel blocks within one head and
// one group, 16-byte vector access of every row); the caller checks h0 / hfin alignment.
bool ssd_supported(const ScanParams& p);
hipError_t launch_ssd(const ScanParams& p, hipStream_t stream);

// dst[0, n) = src[0, n), or zeros when src is null
hipError_t launch_state_copy(const float* src, float* dst, int64_t n, hipStream_t stream);

}  // namespace ssm
