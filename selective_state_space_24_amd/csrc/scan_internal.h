// Internal launch parameters shared by the host dispatch and the gfx950 kernels.
#pragma once
#include <stdint.h>

namespace ssm {

// Channels handled by one workgroup: one channel per lane of a 64-wide wavefront.
constexpr int kChannelsPerGroup = 64;

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
};

}  // namespace ssm
