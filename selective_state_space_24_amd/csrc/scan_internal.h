// Internal launch parameters shared by the host dispatch and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_scan.h"

namespace ssm {

// Channels handled by one workgroup: one channel per lane of a 64-wide wavefront.
constexpr int kChannelsPerGroup = 64;
// Wavefronts per workgroup; they split the states of the workgroup's channels.
constexpr int kWavesPerGroup = 4;
constexpr int kTB = 32;       // time steps per compute tile
constexpr int kLT = 2 * kTB;  // time steps per load tile (128 bytes of bf16 per row); segments
                              // along L start at multiples of it
constexpr int kCkptStep = 8;  // steps between the states the backward checkpoint pass stores
constexpr int kHeadDeltaChunk = 1024;  // steps per partial sum of the head-mode bias gradient
constexpr int kFixCheck = 1024;  // steps between the states a split output pass stores for the
                                 // pass that corrects its later segments (checked against there)
constexpr int kFixMaxChecks = 32;  // stored states per segment at most (the first 32K steps)
constexpr int64_t kFixMinSegment = 32768;  // shortest segment that takes that scheme

constexpr int64_t kCUs = 256;           // compute units of an MI355X
constexpr int64_t kTargetWaves = 2048;  // about two resident wavefronts per SIMD (256 CUs)

// True when `groups` (batch x 64-channel groups) runs the whole sequence in one pass without
// further thought: enough 64-channel, four-wavefront workgroups for three quarters of the
// target waves.
inline bool groups_fill_chip(int64_t groups) {
  return groups * kWavesPerGroup * 4 >= kTargetWaves * 3;
}

// bf16 io with 8 < N <= 16 normally runs the kernel with independent wavefronts (128-channel,
// 8-wavefront workgroups, one per CU). With 64-channel groups for three quarters of the CUs or
// more, but too few 128-channel workgroups to fill the chip, the whole sequence runs in one pass
// in 64-channel workgroups instead: four independent wavefronts in the forward pass, the
// barrier-synchronised kernel's four wavefronts of four states in the backward's checkpoint
// pass. The forward planner and the backward both take this choice from here.
inline bool narrow_one_pass(int64_t groups) {
  return groups * 4 >= kCUs * 3 && !groups_fill_chip(groups);
}

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
  // the independent-wavefront kernel's split: its output pass's zero-start state after every
  // kFixCheck steps of each segment, all 16 padded states, hchk[(((b * dim + d) * nseg + s) *
  // nchk + k) * 16 + n] (16-byte aligned; nullable when nchk == 0)
  float* hchk;
  int64_t nchk;

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
  int32_t narrow_groups;     // bf16 io, 8 < N <= 16: run the kernel with independent wavefronts
                             // in 64-channel workgroups of four, in one pass (chosen by the
                             // segment planner)
  int32_t fix_split;         // the kernel with independent wavefronts, split along L: zero-start
                             // output pass, then the correcting pass (rather than a summary pass
                             // first; chosen by the segment planner)
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
  int32_t vec_out;   // dx, ddelta, dz allow 16-byte stores (16-byte aligned bases, with the
                     // strides of x, delta, z, which vec_io makes multiples of 16 bytes)
  int32_t part_vec;  // the dB, dC partials allow 16-byte stores (aligned bases, L % 4 == 0)
  int32_t head;      // one A per head (the forward's a_mode SSM_A_HEAD)
  int32_t head_ns;   // head mode: states per lane of the reverse kernel (dA_part holds one value
                     // per lane at the first state of each wavefront's block)
  int64_t span;      // head mode: channels per row of ddl_part (gcd(headdim, 64))
  const float* dhfin;  // nullable: gradient of the final state (batch, dim, N)
  float* ddl_part;     // head mode: ddelta before the activation, summed over runs of span
                       // channels, (batch, dim / span, L)
  float* dbias_hpart;  // head mode: (nheads, batch, ceil(L / kHeadDeltaChunk)) partial sums
};
hipError_t launch_bwd(const BwdParams& q, bool bf16, hipStream_t stream);
// the reverse kernel of one A per head, dstate > 16 or the zero-order hold (with its checkpoint
// pass and the head-mode ddelta reduction), per io dtype; launch_bwd adds the reductions
hipError_t launch_bwd_wide_bf16(const BwdParams& q, hipStream_t stream);
hipError_t launch_bwd_wide_f32(const BwdParams& q, hipStream_t stream);
// states per lane of that kernel for dstate N (4, 8 or 16)
inline int bwd_wide_states_per_lane(int64_t N) { return N <= 16 ? 4 : (N <= 32 ? 8 : 16); }
// Chunked matrix form of the head-mode forward pass (bf16 io, MFMA). ssd_supported checks the
// shape and access conditions it needs (dstate 64 or 128, 64-channel blocks within one head and
// one group, 16-byte vector access of every row); the caller checks h0 / hfin alignment.
bool ssd_supported(const ScanParams& p);
hipError_t launch_ssd(const ScanParams& p, hipStream_t stream);

// dst[0, n) = src[0, n), or zeros when src is null
hipError_t launch_state_copy(const float* src, float* dst, int64_t n, hipStream_t stream);
hipError_t launch_wave_simd(int32_t* out, int32_t nworkgroups, hipStream_t stream);
// The forward scan with a complex diagonal A (a_mode SSM_A_COMPLEX): A as (dim, N, 2) fp32
// pairs, B and C with 2N rows per group (real parts, then imaginary), N <= 32, delta * B rule,
// no initial or final state (checked by the caller).
hipError_t launch_complex(const ScanParams& p, bool bf16, hipStream_t stream);

// The forward entry point behind ssm_selective_scan_fwd_ext. `checks` off leaves out the states
// that a split sequence's output pass stores for the correcting pass (a smaller workspace; the
// correcting pass then runs every later segment to its end, with the same results).
// fwd_workspace_bytes is the workspace either way, for a descriptor that check_desc accepts.
size_t fwd_workspace_bytes(const ssm_scan_desc* desc, bool checks);
int fwd_ext(const ssm_scan_desc* desc, const void* x, const void* delta, const float* A,
            const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
            int32_t delta_softplus, void* y, const ssm_scan_ext* ext, void* workspace,
            size_t workspace_bytes, void* stream, bool checks);

}  // namespace ssm
