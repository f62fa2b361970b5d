// gfx950 kernels of the selective-scan backward pass: the gradients of every input.
//
// The pages train the layer end to end and recompute the states in the backward pass rather
// than storing them (page "NL-345", §1 "Hardware-aware Algorithm"). Here:
//   1. a checkpoint pass (the forward kernel without readout) stores the state before every
//      8th step: N fp32 values per channel per 8 steps;
//   2. the backward kernel walks each channel group's 32-step tiles in reverse. A tile is
//      processed in 8-step sub-tiles, last first: a sub-tile starts from its checkpoint (read
//      one sub-tile ahead), its 8 states are recomputed into registers and the reverse
//      recurrence runs over them:
//        gh += gy C;  dC += gy h;  ddelta += gh (a dA h_prev + B x);  da += gh dA h_prev delta;
//        dB += gh delta x;  dx += gh delta B;  gh *= dA
//      (gy = dy silu(z) is the gradient of the ungated readout). As in the forward pass, lane =
//      channel and the four wavefronts split the states, so the per-channel sums over states
//      (ddelta, dx, and the readout needed by dz) are added across wavefronts in LDS, and the
//      per-(t, n) sums over channels (dB, dC) are added over the lanes of each wavefront in
//      wave-private LDS, giving one partial per workgroup;
//   3. reduce kernels add the partials: dB, dC over the workgroups of a batch entry's group,
//      dA, dD, dbias over the batch, in a fixed order (results are deterministic).
// The LDS use (about 74 KB) lets two workgroups share a CU. Arithmetic: fp32. This kernel takes
// diagonal A, dstate <= 16 and the delta * B rule; scan_bwd_wide.h takes every other case and
// shares the reductions below.
#include "scan_bwd_common.h"

namespace ssm {

constexpr int kBT = kTB;            // steps per backward tile (one load of the per-step inputs)
constexpr int kSub = 8;             // steps per sub-tile (their states are held in registers)
constexpr int kSubs = kBT / kSub;   // sub-tiles per tile
static_assert(kSub == kCkptStep, "every sub-tile starts at a checkpoint");
constexpr int kInStride = kBT + 1;  // entries per channel row of the per-step LDS arrays
constexpr int kRedStride = kSub + 1;
// floats per column of the dB/dC lane-sum scratch (64 lanes, padded so that the 16-byte column
// reads of consecutive columns start in different bank groups)
constexpr int kSumStride = 64 + 4;

template <typename IO, int NS, bool GATE>
__global__ void __launch_bounds__(256, 2) bwd_kernel(const BwdParams q) {
  constexpr int NW = kWavesPerGroup;
  constexpr int NT = 64 * NW;
  constexpr int NP = NS * NW;
  constexpr int V = IoTraits<IO>::kVec;
  constexpr int CPT = kBT / V;                      // chunks per channel row of a tile
  constexpr int ITEMS = kChannelsPerGroup * CPT;
  constexpr int IPT = ITEMS / NT;                   // prologue items per thread
  constexpr int RS = NS >= 4 ? 2 : 4;               // steps per dB/dC lane reduction
  constexpr int NV = 2 * NS * RS;                   // dB/dC values per lane per reduction
  static_assert(ITEMS % NT == 0, "prologue items must divide evenly");
  static_assert(NV <= 32 && 64 % NV == 0, "dB/dC reduction layout");

  __shared__ __align__(16) f32x4 s_in[kChannelsPerGroup * kInStride];  // delta, u, gy, x
  __shared__ float s_gz[kChannelsPerGroup * kInStride];                 // dy silu'(z)
  __shared__ __align__(16) float s_B[NP * kBT];
  __shared__ __align__(16) float s_C[NP * kBT];
  __shared__ __align__(16) float s_red[3 * NW * kChannelsPerGroup * kRedStride];

  const ScanParams& p = q.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t wg = blockIdx.x % p.groups_per_batch;
  const int64_t b = blockIdx.x / p.groups_per_batch;
  const int64_t d0 = wg * kChannelsPerGroup;
  const int64_t grp = d0 / (p.dim / p.ngroups);
  const int n0 = w * NS;
  const int64_t L = p.L;
  const bool vec = p.vec_io != 0;
  const IO* X = static_cast<const IO*>(p.x);
  const IO* DL = static_cast<const IO*>(p.delta);
  const IO* Z = static_cast<const IO*>(p.z);
  const IO* DY = static_cast<const IO*>(q.dy);
  const IO* Bg = static_cast<const IO*>(p.B) + b * p.B_sb + grp * p.B_sg;
  const IO* Cg = static_cast<const IO*>(p.C) + b * p.C_sb + grp * p.C_sg;

  // this lane's channel and states
  const int64_t d = d0 + lane;
  const bool live = d < p.dim;
  float ap[NS], an[NS];  // a * log2(e) for exp2, and a itself
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    an[j] = (live && n0 + j < p.N) ? p.A[d * p.N + n0 + j] : 0.0f;
    ap[j] = an[j] * kLog2e;
  }

  // the epilogue's item: channel er, steps [2 * eq, 2 * eq + 2) of each sub-tile
  const int er = tid >> 2, eq = tid & 3;
  const int64_t ed = d0 + er;
  const bool elive = ed < p.dim;
  const float eD = (elive && p.D) ? p.D[ed] : 0.0f;
  float dD_acc = 0.0f, dbias_acc = 0.0f;

  float gh[NS], da[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    gh[j] = (q.dhfin && live && n0 + j < p.N) ? q.dhfin[(b * p.dim + d) * p.N + n0 + j] : 0.0f;
    da[j] = 0.0f;
  }

  for (int64_t tile = (L + kBT - 1) / kBT - 1; tile >= 0; --tile) {
    const int64_t t0 = tile * kBT;
    const int lt_len = (int)min<int64_t>(kBT, L - t0);

    // ---- prologue: per (channel, step) values of the tile into LDS; padding steps are zero
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int r = item / CPT, tl = (item % CPT) * V;
      const int64_t dd = d0 + r;
      const int64_t dv = min(dd, p.dim - 1);
      const int cnt = dd < p.dim ? max(0, min(V, lt_len - tl)) : 0;
      float xv[V], dv_raw[V], zv[V], gv[V];
      load_chunk<IO, true>(X + b * p.x_sb + dv * p.x_sd, t0 + tl, cnt, vec, xv);
      load_chunk<IO, true>(DL + b * p.dl_sb + dv * p.dl_sd, t0 + tl, cnt, vec, dv_raw);
      load_chunk<IO, true>(DY + b * p.y_sb + dv * p.y_sd, t0 + tl, cnt, vec, gv);
      if constexpr (GATE) load_chunk<IO, true>(Z + b * p.z_sb + dv * p.z_sd, t0 + tl, cnt, vec, zv);
      const float bias = (dd < p.dim && p.delta_bias) ? p.delta_bias[dv] : 0.0f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float dl = 0.0f, u = 0.0f, gy = 0.0f, xx = 0.0f, gzf = 0.0f;
        if (e < cnt) {
          const float v = dv_raw[e] + bias;
          dl = p.softplus ? softplus_f32(v) : v;
          xx = xv[e];
          u = dl * xx;
          gy = gv[e];
          if constexpr (GATE) {
            const float zz = zv[e];
            const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz * kLog2e));
            gzf = gv[e] * s * fmaf(zz, 1.0f - s, 1.0f);
            gy = gv[e] * zz * s;
          }
        }
        s_in[r * kInStride + tl + e] = f32x4{dl, u, gy, xx};
        s_gz[r * kInStride + tl + e] = gzf;
      }
    }
    for (int i = tid; i < NP * kBT; i += NT) {
      const int n = i / kBT, t = i % kBT;
      const bool on = n < p.N && t < lt_len;
      s_B[n * kBT + t] = on ? to_f32(Bg[n * p.B_sn + t0 + t]) : 0.0f;
      s_C[n * kBT + t] = on ? to_f32(Cg[n * p.C_sn + t0 + t]) : 0.0f;
    }
    // the checkpoints of the tile's sub-tiles (channel-contiguous); the last sub-tile's is
    // read now and each earlier one while the sub-tile after it runs. A sub-tile entirely past
    // L has none: its steps are padding, and it starts from 0.
    const float* ck = p.ckpt + ((b * p.ntiles + tile * kSubs) * p.N + n0) * p.dim + (live ? d : 0);
    auto load_ck = [&](int k, float (&hv)[NS]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NS; ++j)
        hv[j] = (live && n0 + j < p.N && t0 + k * kSub < L) ? ck[(k * p.N + j) * p.dim] : 0.0f;
    };
    float hnext[NS];
    load_ck(kSubs - 1, hnext);
    __syncthreads();

    // ---- sub-tiles, last first
#pragma unroll 1
    for (int k = kSubs - 1; k >= 0; --k) {
      const int tb = k * kSub;
      float hsk[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) hsk[j] = hnext[j];
      if (k > 0) load_ck(k - 1, hnext);
      // recompute the sub-tile's states (after each step) and the readout partials
      float hh[kSub][NS];
      float yp[kSub];
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        const f32x4 in = s_in[lane * kInStride + tb + i];
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float prev = i == 0 ? hsk[j] : hh[i - 1][j];
          hh[i][j] = fmaf(__builtin_amdgcn_exp2f(in.x * ap[j]), prev,
                          in.y * s_B[(n0 + j) * kBT + tb + i]);
          acc = fmaf(s_C[(n0 + j) * kBT + tb + i], hh[i][j], acc);
        }
        yp[i] = acc;
      }
      // reverse recurrence over the sub-tile
      float gdel[kSub];
      // wavefront w's block of s_red (its three partial arrays) doubles as its private scratch
      // for the dB/dC lane sums, which use its first 64 (NV + 1) floats: that is within the
      // first two arrays, so the third (rx, the dx partials) is written as the steps go
      float* scratch = s_red + w * 3 * kChannelsPerGroup * kRedStride;
      float* rx = s_red + ((w * 3 + 2) * kChannelsPerGroup + lane) * kRedStride;
      static_assert(NV * kSumStride <= 2 * kChannelsPerGroup * kRedStride,
                    "lane-sum scratch must stay clear of the dx partials");
      // the scratch is column-major: value v of lane l at scratch[v * kSumStride + l], with v =
      // [tensor (dC, dB)][state j][step e]
      float* red = scratch + lane;
#pragma unroll
      for (int i4 = kSub - RS; i4 >= 0; i4 -= RS) {
#pragma unroll
        for (int e = RS - 1; e >= 0; --e) {
          const int i = i4 + e;
          const int t = tb + i;
          const f32x4 in = s_in[lane * kInStride + t];
          const float dl = in.x, u = in.y, gy = in.z, xx = in.w;
          // ddelta and dx need sum_j gh_j (h_prev,j dA_j a_j + B_j x) and sum_j gh_j delta B_j:
          // both are taken as sum_j gh_j h_prev,j dA_j a_j plus x and delta times sum_j gh_j B_j
          float gd = 0.0f, sb = 0.0f;
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const float Bv = s_B[(n0 + j) * kBT + t];
            const float Cv = s_C[(n0 + j) * kBT + t];
            gh[j] = fmaf(gy, Cv, gh[j]);
            red[(j * RS + e) * kSumStride] = gy * hh[i][j];        // dC
            const float dA = __builtin_amdgcn_exp2f(dl * ap[j]);
            const float hp = i == 0 ? hsk[j] : hh[i - 1][j];
            const float gt = gh[j] * (hp * dA);
            gd = fmaf(gt, an[j], gd);
            da[j] = fmaf(gt, dl, da[j]);
            red[(RS * NS + j * RS + e) * kSumStride] = gh[j] * u;  // dB
            sb = fmaf(gh[j], Bv, sb);
            gh[j] *= dA;
          }
          gdel[i] = fmaf(xx, sb, gd);
          rx[i] = dl * sb;
        }
        // sum the RS steps' dC, dB over the wavefront's lanes (channels) via wave-private LDS
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane sums value col = lane % NV of the NV lanes part * NV .. + NV (four 16-byte reads
        // of one column); the 64 / NV lanes of a column then combine across lanes
        const int col = lane % NV, part = lane / NV;
        float sum;
        {
          const f32x4* src = reinterpret_cast<const f32x4*>(scratch + col * kSumStride + part * NV);
          f32x4 acc4 = src[0];
#pragma unroll
          for (int r4 = 1; r4 < NV / 4; ++r4) acc4 += src[r4];
          sum = (acc4.x + acc4.y) + (acc4.z + acc4.w);
        }
#pragma unroll
        for (int off = NV; off < 64; off <<= 1) sum = xor_sum(sum, off);
        if (lane < NV) {
          const int tensor = col / (RS * NS), j = (col / RS) % NS, e = col % RS;
          const int64_t t = t0 + tb + i4 + e;
          if (n0 + j < p.N && t < L) {
            float* dst = tensor == 0 ? q.dC_part : q.dB_part;
            dst[((b * p.groups_per_batch + wg) * p.N + n0 + j) * L + t] = sum;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      // per-channel partial sums over this wavefront's states
      {
        float* ry = s_red + ((w * 3 + 0) * kChannelsPerGroup + lane) * kRedStride;
        float* rg = s_red + ((w * 3 + 1) * kChannelsPerGroup + lane) * kRedStride;
#pragma unroll
        for (int i = 0; i < kSub; ++i) {
          ry[i] = yp[i];
          rg[i] = gdel[i];
        }
      }
      __syncthreads();
      // epilogue: add the wavefronts' partials; dx, ddelta, dz for 2 steps of one channel
      {
        float vx[2], vd[2], vz[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = eq * 2 + e;
          const int t = tb + i;
          float ys = 0.0f, gds = 0.0f, gxsum = 0.0f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) {
            ys += s_red[((ww * 3 + 0) * kChannelsPerGroup + er) * kRedStride + i];
            gds += s_red[((ww * 3 + 1) * kChannelsPerGroup + er) * kRedStride + i];
            gxsum += s_red[((ww * 3 + 2) * kChannelsPerGroup + er) * kRedStride + i];
          }
          const f32x4 in = s_in[er * kInStride + t];
          const float y = fmaf(eD, in.w, ys);
          vz[e] = s_gz[er * kInStride + t] * y;
          vx[e] = fmaf(in.z, eD, gxsum);
          vd[e] = gds * (p.softplus ? sigmoid_from_softplus(in.x) : 1.0f);
          dD_acc = fmaf(in.z, in.w, dD_acc);
          dbias_acc += vd[e];
        }
        if (elive) {
          const int64_t tt = t0 + tb + eq * 2;
          IO* dxr = static_cast<IO*>(q.dx) + b * p.x_sb + ed * p.x_sd;
          IO* ddr = static_cast<IO*>(q.ddelta) + b * p.dl_sb + ed * p.dl_sd;
          IO* dzr = GATE ? static_cast<IO*>(q.dz) + b * p.z_sb + ed * p.z_sd : nullptr;
          if (q.pair_out && tt + 1 < L) {
            // tt is even: both steps in one store per tensor
            store_pair(dxr + tt, vx[0], vx[1]);
            store_pair(ddr + tt, vd[0], vd[1]);
            if constexpr (GATE) store_pair(dzr + tt, vz[0], vz[1]);
          } else {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              if (tt + e < L) {
                store_elem(dxr + tt + e, vx[e]);
                store_elem(ddr + tt + e, vd[e]);
                if constexpr (GATE) store_elem(dzr + tt + e, vz[e]);
              }
            }
          }
        }
      }
      __syncthreads();  // s_red is reused by the next sub-tile
    }
  }

  // ---- per-workgroup partials of the batch-summed gradients, and dh0
  if (live) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (n0 + j >= p.N) continue;
      q.dA_part[(b * p.dim + d) * p.N + n0 + j] = da[j];
      if (q.dh0) q.dh0[(b * p.dim + d) * p.N + n0 + j] = gh[j];
    }
  }
  dD_acc += __shfl_xor(dD_acc, 1);
  dD_acc += __shfl_xor(dD_acc, 2);
  dbias_acc += __shfl_xor(dbias_acc, 1);
  dbias_acc += __shfl_xor(dbias_acc, 2);
  if (elive && eq == 0) {
    q.dD_part[b * p.dim + ed] = dD_acc;
    q.dbias_part[b * p.dim + ed] = dbias_acc;
  }
}

// dB, dC: the sum over the workgroups of each (batch entry, group), one thread per (b, g, n, t)
__global__ void __launch_bounds__(256) bwd_reduce_bc(const BwdParams q) {
  const ScanParams& p = q.f;
  const int64_t L = p.L, N = p.N;
  const int64_t total = p.batch * p.ngroups * N * L;
  const int64_t wg_per_group = p.groups_per_batch / p.ngroups;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t t = i % L, n = (i / L) % N, g = (i / (L * N)) % p.ngroups, b = i / (L * N * p.ngroups);
    float sb = 0.0f, sc = 0.0f;
    for (int64_t k = 0; k < wg_per_group; ++k) {
      const int64_t idx = ((b * p.groups_per_batch + g * wg_per_group + k) * N + n) * L + t;
      sb += q.dB_part[idx];
      sc += q.dC_part[idx];
    }
    q.dB[b * p.B_sb + g * p.B_sg + n * p.B_sn + t] = sb;
    q.dC[b * p.C_sb + g * p.C_sg + n * p.C_sn + t] = sc;
  }
}

// dA, dD, dbias: the sums over the batch, one thread per (d, n)
__global__ void __launch_bounds__(256) bwd_reduce_params(const BwdParams q) {
  const ScanParams& p = q.f;
  const int64_t N = p.N;
  const int64_t total = p.dim * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int64_t b = 0; b < p.batch; ++b) s += q.dA_part[b * total + i];
    q.dA[i] = s;
    if (i % N == 0) {
      const int64_t d = i / N;
      float sd = 0.0f, sbias = 0.0f;
      for (int64_t b = 0; b < p.batch; ++b) {
        sd += q.dD_part[b * p.dim + d];
        sbias += q.dbias_part[b * p.dim + d];
      }
      if (q.dD) q.dD[d] = sd;
      if (q.dbias) q.dbias[d] = sbias;
    }
  }
}

// Head mode: dA[h] (sum over batch entries, the head's channels and the wavefronts' state
// blocks), dbias[h] (sum over batch entries and chunks) and dD[d] (sum over batch entries).
__global__ void __launch_bounds__(256) bwd_reduce_params_head(const BwdParams q) {
  const ScanParams& p = q.f;
  const int64_t nheads = p.dim / p.headdim;
  const int64_t nchunks = (p.L + kHeadDeltaChunk - 1) / kHeadDeltaChunk;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < p.dim && q.dD) {
    float s = 0.0f;
    for (int64_t b = 0; b < p.batch; ++b) s += q.dD_part[b * p.dim + i];
    q.dD[i] = s;
  }
  if (i < nheads) {
    float sa = 0.0f;
    for (int64_t b = 0; b < p.batch; ++b)
      for (int64_t d = i * p.headdim; d < (i + 1) * p.headdim; ++d)
        for (int64_t n = 0; n < p.N; n += q.head_ns) sa += q.dA_part[(b * p.dim + d) * p.N + n];
    q.dA[i] = sa;
    if (q.dbias) {
      float sb = 0.0f;
      for (int64_t b = 0; b < p.batch; ++b)
        for (int64_t c = 0; c < nchunks; ++c) sb += q.dbias_hpart[(i * p.batch + b) * nchunks + c];
      q.dbias[i] = sb;
    }
  }
}

// dB, dC (over the workgroups of each batch entry's group) and the parameter gradients (over
// the batch; in head mode also over each head's channels), all in a fixed order
static hipError_t bwd_reductions(const BwdParams& q, hipStream_t stream) {
  const ScanParams& p = q.f;
  const int64_t nbc = p.batch * p.ngroups * p.N * p.L;
  const int64_t bbc = (nbc + 255) / 256;
  const unsigned gbc = (unsigned)(bbc < 65536 ? bbc : 65536);
  hipLaunchKernelGGL(bwd_reduce_bc, dim3(gbc > 0 ? gbc : 1), dim3(256), 0, stream, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (q.head) {
    hipLaunchKernelGGL(bwd_reduce_params_head, dim3((unsigned)((p.dim + 255) / 256)), dim3(256),
                       0, stream, q);
    return hipGetLastError();
  }
  const int64_t np = p.dim * p.N;
  const int64_t bp = (np + 255) / 256;
  hipLaunchKernelGGL(bwd_reduce_params, dim3((unsigned)(bp < 65536 ? bp : 65536)), dim3(256), 0,
                     stream, q);
  return hipGetLastError();
}

template <typename IO, int NS>
static hipError_t bwd_cfg(const BwdParams& q, hipStream_t stream) {
  const ScanParams& p = q.f;
  const int64_t groups = p.batch * p.groups_per_batch;
  // 1. checkpoints (bf16 io with 8 < N <= 16: the kernel with independent wavefronts, except
  // where the forward's planner takes the state-split kernel, state_split_one_pass: then the
  // barrier-synchronised kernel's four wavefronts of four states)
  auto four_wave_ckpt = [&]() {
    hipLaunchKernelGGL((scan_fwd_kernel<IO, NS, kWavesPerGroup, false, false, false, false, true>),
                       dim3((unsigned)groups, 1), dim3(64 * kWavesPerGroup), 0, stream,
                       static_cast<const IO*>(p.x), static_cast<const IO*>(p.delta),
                       static_cast<const IO*>(p.B), static_cast<const IO*>(p.C),
                       static_cast<const IO*>(nullptr), static_cast<IO*>(nullptr), p.A, p.D,
                       p.delta_bias, nullptr, nullptr, p);
  };
  if constexpr (NS == 4 && WaveIo<IO>::value) {
    if (!state_split_one_pass(groups)) {
      const unsigned wg = (unsigned)(p.batch * ((p.dim + kWaveGroupChannels - 1) / kWaveGroupChannels));
      hipLaunchKernelGGL((scan_fwd_wave_kernel<IO, false, false, false, kWaveCkpt>), dim3(wg, 1),
                         dim3(64 * kWaveGroupWaves), 0, stream, static_cast<const IO*>(p.x),
                         static_cast<const IO*>(p.delta), static_cast<const IO*>(p.B),
                         static_cast<const IO*>(p.C), static_cast<const IO*>(nullptr),
                         static_cast<IO*>(nullptr), p.A, p.D, p.delta_bias, nullptr, nullptr, p);
    } else {
      four_wave_ckpt();
    }
  } else {
    four_wave_ckpt();
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. the reverse pass
  if (p.z)
    hipLaunchKernelGGL((bwd_kernel<IO, NS, true>), dim3((unsigned)groups), dim3(256), 0, stream, q);
  else
    hipLaunchKernelGGL((bwd_kernel<IO, NS, false>), dim3((unsigned)groups), dim3(256), 0, stream, q);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. reductions
  return bwd_reductions(q, stream);
}

template <typename IO>
static hipError_t bwd_n(const BwdParams& q, hipStream_t stream) {
  const int64_t N = q.f.N;
  if (N <= 4) return bwd_cfg<IO, 1>(q, stream);
  if (N <= 8) return bwd_cfg<IO, 2>(q, stream);
  return bwd_cfg<IO, 4>(q, stream);  // N <= 16 (checked by the caller)
}

hipError_t launch_bwd(const BwdParams& q, bool bf16, hipStream_t stream) {
  // one A per head, dstate above 16 or the zero-order hold: the kernel of scan_bwd_wide.h
  if (q.head || q.f.zoh || q.f.N > 16) {
    const hipError_t e = bf16 ? launch_bwd_wide_bf16(q, stream) : launch_bwd_wide_f32(q, stream);
    if (e != hipSuccess) return e;
    return bwd_reductions(q, stream);
  }
  return bf16 ? bwd_n<bf16_bits>(q, stream) : bwd_n<float>(q, stream);
}

}  // namespace ssm
