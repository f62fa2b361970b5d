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
//      wave-private LDS, giving one partial per workgroup. Outputs wait in LDS until the tile is
//      done (dx, ddelta, dz in the slots of the consumed inputs, the dB/dC partials in a tile
//      buffer), then in registers, and leave in whole 16-byte pieces while the next tile runs;
//      for bf16 the next tile's inputs are loaded while the tile runs;
//   3. reduce kernels add the partials: dB, dC over the workgroups of a batch entry's group,
//      dA, dD, dbias over the batch, in a fixed order (results are deterministic).
// The LDS use (under 80 KB) lets two workgroups share a CU. Arithmetic: fp32. This kernel takes
// diagonal A, dstate <= 16 and the delta * B rule; scan_bwd_wide.h takes every other case and
// shares the reductions below.
#include "scan_bwd_common.h"

namespace ssm {

constexpr int kBT = kTB;            // steps per backward tile (one load of the per-step inputs)
constexpr int kSub = 8;             // steps per sub-tile (their states are held in registers)
constexpr int kSubs = kBT / kSub;   // sub-tiles per tile
static_assert(kSub == kCkptStep, "every sub-tile starts at a checkpoint");
// The per-step LDS entries of a channel row: step t sits at in_col(t) = t + 2 (t / 8), two spare
// entries after every 8 steps, in rows of an odd kInStride entries. A wavefront that reads one
// step of 64 rows (lane = row) then hits 8 different 16-byte bank groups in every 8 lanes, and so
// does one that writes 16-byte chunks of 16 rows, four lanes to a row (a chunk of 8 steps starts
// 10 entries after the one before it).
constexpr int kInStride = kBT + 7;
static_assert(kInStride % 2 == 1 && kInStride >= kBT + 2 * (kBT / 8 - 1), "row layout");
__device__ __forceinline__ constexpr int in_col(int t) { return t + 2 * (t >> 3); }
constexpr int kRedStride = kSub + 1;

// NS consecutive floats of LDS at p (aligned to NS floats) as one read
template <int NS>
__device__ __forceinline__ void lds_states(const float* p, float (&v)[NS]) {
  if constexpr (NS == 4) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else if constexpr (NS == 2) {
    const float2 q = *reinterpret_cast<const float2*>(p);
    v[0] = q.x; v[1] = q.y;
  } else {
    v[0] = p[0];
  }
}

template <typename IO, int NS, bool GATE>
__global__ void __launch_bounds__(256, 2) bwd_kernel(const BwdParams q) {
  constexpr int NW = kWavesPerGroup;
  constexpr int NT = 64 * NW;
  constexpr int NP = NS * NW;
  constexpr int V = IoTraits<IO>::kVec;
  constexpr int CPT = kBT / V;                      // chunks per channel row of a tile
  constexpr int ITEMS = kChannelsPerGroup * CPT;
  constexpr int IPT = ITEMS / NT;                   // prologue items per thread
  constexpr int BCI = (NP * kBT + NT - 1) / NT;     // B (and C) elements per thread per tile
  // the next tile's inputs are loaded while this tile runs where they take few registers (one
  // 16-byte chunk per tensor per thread); otherwise right before they are needed
  constexpr bool PREFETCH = IPT == 1;
  constexpr int M = 2 * NS;                         // dB/dC values per lane per step
  constexpr int G = 64 / M;                         // lanes that end up holding each sum
  static_assert(ITEMS % NT == 0, "prologue items must divide evenly");

  __shared__ __align__(16) f32x4 s_in[kChannelsPerGroup * kInStride];  // delta, gz, gy, x
  // B and C step-major: a wavefront's NS states of a step are one aligned vector. Steps are
  // kBCRow floats apart, an odd multiple of 4, so that the fill's stores along the steps of a
  // state spread over 8 bank groups
  constexpr int kBCRow = NP % 8 == 0 ? NP + 4 : NP;
  __shared__ __align__(16) float s_B[kBT * kBCRow];
  __shared__ __align__(16) float s_C[kBT * kBCRow];
  __shared__ __align__(16) float s_red[3 * NW * kChannelsPerGroup * kRedStride];
  // the tile's dC, dB partials, (tensor, n, t): rows of kDbcRow floats, the dB rows 16 floats
  // further on, so that the eight sums a wavefront stores per step (four states of each tensor)
  // fall in eight different LDS banks
  constexpr int kDbcRow = kBT + 4, kDbcTensor = NP * kDbcRow + 16;
  __shared__ __align__(16) float s_dbc[2 * kDbcTensor];

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
  float ap[NS];  // a * log2(e), for exp2
#pragma unroll
  for (int j = 0; j < NS; ++j) ap[j] = ((live && n0 + j < p.N) ? p.A[d * p.N + n0 + j] : 0.0f) * kLog2e;

  // the epilogue's item: channel er (the lane), steps [2 * eq, 2 * eq + 2) of each sub-tile (eq
  // the wavefront), so that a wavefront's reads of the per-channel partials and of the step
  // slots run along the channels, whose LDS rows are padded to different banks
  const int er = tid & 63, eq = tid >> 6;
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

  // ---- a tile's per-step inputs: raw 16-byte chunks (x, delta, dy, z) of this thread's prologue
  // items and its B, C elements; then converted into LDS (padding steps are zero). With the
  // prefetch, an odd tile's chunks are loaded together with those of the even tile before it:
  // the two share each 128-byte line of a bf16 row, which is then read whole. An odd tile's
  // chunks are held in raw_odd, an even tile's in raw_even; loads go straight into them and
  // nothing copies them, since a copy of a register a load is still writing waits for that
  // load.
  struct Items {
    u32x4 c[IPT][4];  // per item: x, delta, dy, z
  };
  Items raw_odd, raw_even;
  IO rb[BCI], rc[BCI];
  auto load_items = [&](int64_t tile) __attribute__((always_inline)) {
    const int64_t t0 = tile * kBT;
    const int lt_len = (int)min<int64_t>(kBT, L - t0);
    Items o;
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int r = item / CPT, tl = (item % CPT) * V;
      const int64_t dd = d0 + r;
      const int64_t dv = min(dd, p.dim - 1);
      const int cnt = dd < p.dim ? max(0, min(V, lt_len - tl)) : 0;
      o.c[it][0] = load_raw16<IO>(X + b * p.x_sb + dv * p.x_sd, t0 + tl, cnt, vec);
      o.c[it][1] = load_raw16<IO>(DL + b * p.dl_sb + dv * p.dl_sd, t0 + tl, cnt, vec);
      o.c[it][2] = load_raw16<IO>(DY + b * p.y_sb + dv * p.y_sd, t0 + tl, cnt, vec);
      o.c[it][3] = GATE ? load_raw16<IO>(Z + b * p.z_sb + dv * p.z_sd, t0 + tl, cnt, vec)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    return o;
  };
  auto issue = [&](int64_t tile, bool pair) __attribute__((always_inline)) {
    const int64_t t0 = tile * kBT;
    const int lt_len = (int)min<int64_t>(kBT, L - t0);
    if (!PREFETCH) {
      raw_even = load_items(tile);
    } else if (tile & 1) {
      raw_odd = load_items(tile);
      if (pair) raw_even = load_items(tile - 1);
    } else if (!pair) {
      raw_even = load_items(tile);  // an even tile with no odd one after it
    }  // (else an even tile loaded with the odd one after it)
#pragma unroll
    for (int k = 0; k < BCI; ++k) {
      const int i = tid + k * NT;
      const int n = i / kBT, t = i % kBT;
      const bool on = i < NP * kBT && n < p.N && t < lt_len;
      rb[k] = on ? Bg[n * p.B_sn + t0 + t] : IO(0);
      rc[k] = on ? Cg[n * p.C_sn + t0 + t] : IO(0);
    }
  };
  // the delta bias of each prologue item's channel, read once: inside the tile loop the compiler
  // would read it again every tile (the loop's stores might alias it) and wait for it
  float item_bias[IPT];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int64_t dd = d0 + (tid + it * NT) / CPT;
    item_bias[it] = (dd < p.dim && p.delta_bias) ? p.delta_bias[dd] : 0.0f;
  }
  auto fill = [&](int64_t tile) __attribute__((always_inline)) {
    const int64_t t0 = tile * kBT;
    const int lt_len = (int)min<int64_t>(kBT, L - t0);
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int r = item / CPT, tl = (item % CPT) * V;
      const int64_t dd = d0 + r;
      const int cnt = dd < p.dim ? max(0, min(V, lt_len - tl)) : 0;
      const float bias = item_bias[it];
      // this tile's chunks (both sets are complete here: the other one was loaded with them or
      // before them)
      const bool odd = PREFETCH && (tile & 1);
      u32x4 cw[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // a select of the two values (of two lvalues it would select an address, and the
        // chunks would go to memory)
        const u32x4 vo = raw_odd.c[it][c], ve = raw_even.c[it][c];
        cw[c] = odd ? vo : ve;
      }
      float xv[V], dv_raw[V], gv[V], zv[V];
      unpack16<IO>(cw[0], xv);
      unpack16<IO>(cw[1], dv_raw);
      unpack16<IO>(cw[2], gv);
      if constexpr (GATE) unpack16<IO>(cw[3], zv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float dl = 0.0f, gy = 0.0f, xx = 0.0f, gzf = 0.0f;
        if (e < cnt) {
          const float v = dv_raw[e] + bias;
          dl = p.softplus ? softplus_f32(v) : v;
          xx = xv[e];
          gy = gv[e];
          if constexpr (GATE) {
            const float zz = zv[e];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz * kLog2e));
            gzf = gv[e] * sg * fmaf(zz, 1.0f - sg, 1.0f);
            gy = gv[e] * zz * sg;
          }
        }
        s_in[r * kInStride + in_col(tl + e)] = f32x4{dl, gzf, gy, xx};
      }
    }
#pragma unroll
    for (int k = 0; k < BCI; ++k) {
      const int i = tid + k * NT;
      if (i < NP * kBT) {
        s_B[(i % kBT) * kBCRow + i / kBT] = to_f32(rb[k]);
        s_C[(i % kBT) * kBCRow + i / kBT] = to_f32(rc[k]);
      }
    }
  };

  const int64_t ntile = (L + kBT - 1) / kBT;
  // the checkpoints of a tile's sub-tiles (channel-contiguous). A sub-tile entirely past L has
  // none: its steps are padding, and it starts from 0.
  auto load_ck = [&](int64_t tile, int k, float (&hv)[NS]) __attribute__((always_inline)) {
    const float* ck = p.ckpt + ((b * p.ntiles + tile * kSubs) * p.N + n0) * p.dim + (live ? d : 0);
#pragma unroll
    for (int j = 0; j < NS; ++j)
      hv[j] = (live && n0 + j < p.N && tile * kBT + k * kSub < L) ? ck[(k * p.N + j) * p.dim] : 0.0f;
  };

  // A tile's outputs leave from registers while the next tile runs: its dx, ddelta, dz (one
  // 16-byte word each per prologue item) and its dB, dC partials (one 4-float piece per thread).
  // The stores are issued after the next tile's inputs have arrived, and every load a wait
  // is needed for soon is issued before them: a wait for a load also waits for every store
  // issued before it, so this keeps the stores' latency out of the waits.
  constexpr int PIECES = 2 * NP * kBT / 4;
  static_assert(PIECES <= NT && PIECES % 64 == 0, "at most one partial piece per thread");
  u32x4 out_w[IPT][3];
  f32x4 out_part = {0.0f, 0.0f, 0.0f, 0.0f};
  // both partial arrays' addresses as values, selected per lane below (a select between the
  // two argument fields would load the chosen one from the argument segment, and wait for it)
  const uint64_t dC_base = reinterpret_cast<uint64_t>(q.dC_part);
  const uint64_t dB_base = reinterpret_cast<uint64_t>(q.dB_part);
  auto gather_outputs = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int r = item / CPT, tl = (item % CPT) * V;
      float vx[V], vd[V], vz[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const f32x4 o = s_in[r * kInStride + in_col(tl + e)];
        vx[e] = o.x;
        vd[e] = o.y;
        vz[e] = o.z;
      }
      out_w[it][0] = pack16<IO>(vx);
      out_w[it][1] = pack16<IO>(vd);
      out_w[it][2] = pack16<IO>(vz);
    }
    if (tid < PIECES) {
      const int tensor = tid / (NP * kBT / 4), n = (tid / (kBT / 4)) % NP, tq = (tid % (kBT / 4)) * 4;
      out_part = *reinterpret_cast<const f32x4*>(s_dbc + tensor * kDbcTensor + n * kDbcRow + tq);
    }
  };
  auto put_outputs = [&](int64_t tile) __attribute__((always_inline)) {
    const int64_t t0 = tile * kBT;
    const int lt_len = (int)min<int64_t>(kBT, L - t0);
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int r = item / CPT, tl = (item % CPT) * V;
      const int64_t dd = d0 + r;
      const int cnt = dd < p.dim ? max(0, min(V, lt_len - tl)) : 0;
      if (cnt > 0) {
        const bool full = q.vec_out != 0;
        store_raw16<IO>(static_cast<IO*>(q.dx) + b * p.x_sb + dd * p.x_sd, t0 + tl, cnt, full,
                        out_w[it][0]);
        store_raw16<IO>(static_cast<IO*>(q.ddelta) + b * p.dl_sb + dd * p.dl_sd, t0 + tl, cnt,
                        full, out_w[it][1]);
        if constexpr (GATE)
          store_raw16<IO>(static_cast<IO*>(q.dz) + b * p.z_sb + dd * p.z_sd, t0 + tl, cnt, full,
                          out_w[it][2]);
      }
    }
    if (tid < PIECES) {
      const int tensor = tid / (NP * kBT / 4), n = (tid / (kBT / 4)) % NP, tq = (tid % (kBT / 4)) * 4;
      const int cnt = n < p.N ? max(0, min(4, lt_len - tq)) : 0;
      float* dst = reinterpret_cast<float*>(tensor == 0 ? dC_base : dB_base) +
                   ((b * p.groups_per_batch + wg) * p.N + n) * L + t0 + tq;
      if (q.part_vec && cnt == 4) {
        *reinterpret_cast<f32x4*>(dst) = out_part;
      } else {
        const float pv[4] = {out_part.x, out_part.y, out_part.z, out_part.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < cnt) dst[e] = pv[e];
      }
    }
  };

  // tile pairs (2m, 2m + 1) share their 128-byte lines; the last tile is alone if it is even
  issue(ntile - 1, (ntile - 1) & 1);
  // the start state of the tile's last sub-tile, read one sub-tile ahead like the others
  float hnext[NS];
  load_ck(ntile - 1, kSubs - 1, hnext);
  for (int64_t tile = ntile - 1; tile >= 0; --tile) {
    const int lt_len = (int)min<int64_t>(kBT, L - tile * kBT);
    fill(tile);
    if (tile + 1 < ntile) put_outputs(tile + 1);
    __syncthreads();
    if (PREFETCH && tile > 0) issue(tile - 1, true);

    // wavefront w's per-channel partial sums over its states: readout (ry), ddelta (rg), dx (rx)
    float* ry = s_red + ((w * 3 + 0) * kChannelsPerGroup + lane) * kRedStride;
    float* rg = s_red + ((w * 3 + 1) * kChannelsPerGroup + lane) * kRedStride;
    float* rx = s_red + ((w * 3 + 2) * kChannelsPerGroup + lane) * kRedStride;

    // ---- sub-tiles, last first
#pragma unroll 1
    for (int k = kSubs - 1; k >= 0; --k) {
      const int tb = k * kSub;
      float hsk[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) hsk[j] = hnext[j];
      // the next sub-tile's start state: this tile's, or the last one of the tile before
      if (k > 0) load_ck(tile, k - 1, hnext);
      else if (tile > 0) load_ck(tile - 1, kSubs - 1, hnext);
      // recompute the sub-tile's states (after each step), their decays and the readout partials
      float hh[kSub][NS], dAk[kSub][NS];
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        const f32x4 in = s_in[lane * kInStride + in_col(tb + i)];
        const float u = in.x * in.w;
        float Bv[NS], Cv[NS];
        lds_states<NS>(s_B + (tb + i) * kBCRow + n0, Bv);
        lds_states<NS>(s_C + (tb + i) * kBCRow + n0, Cv);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float prev = i == 0 ? hsk[j] : hh[i - 1][j];
          dAk[i][j] = __builtin_amdgcn_exp2f(in.x * ap[j]);
          hh[i][j] = fmaf(dAk[i][j], prev, u * Bv[j]);
          acc = fmaf(Cv[j], hh[i][j], acc);
        }
        ry[i] = acc;
      }
      // reverse recurrence over the sub-tile
#pragma unroll
      for (int i = kSub - 1; i >= 0; --i) {
        const int t = tb + i;
        const f32x4 in = s_in[lane * kInStride + in_col(t)];
        const float dl = in.x, gy = in.z, xx = in.w;
        const float u = dl * xx;
        // ddelta and dx need sum_j gh_j (h_prev,j dA_j a_j + B_j x) and sum_j gh_j delta B_j:
        // both are taken as sum_j gh_j h_prev,j dA_j a_j plus x and delta times sum_j gh_j B_j;
        // the first sum is formed with a_j log2(e) and scaled by ln 2 once
        float gd = 0.0f, sb = 0.0f;
        float dbc[M];  // this lane's (channel's) terms of dC_j, dB_j at step t
        float Bv[NS], Cv[NS];
        lds_states<NS>(s_B + t * kBCRow + n0, Bv);
        lds_states<NS>(s_C + t * kBCRow + n0, Cv);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          gh[j] = fmaf(gy, Cv[j], gh[j]);
          dbc[j] = gy * hh[i][j];
          const float dA = dAk[i][j];
          const float hp = i == 0 ? hsk[j] : hh[i - 1][j];
          const float gt = gh[j] * (hp * dA);
          gd = fmaf(gt, ap[j], gd);
          da[j] = fmaf(gt, dl, da[j]);
          dbc[NS + j] = gh[j] * u;
          sb = fmaf(gh[j], Bv[j], sb);
          gh[j] *= dA;
        }
        rg[i] = fmaf(xx, sb, gd * kLn2);
        rx[i] = dl * sb;
        // dC_j, dB_j summed over the wavefront's channels, in registers
        const float tot = lane_sums<M>(dbc);
        if ((lane & (G - 1)) == 0) {
          const int v = lane / G;
          s_dbc[(v / NS) * kDbcTensor + (n0 + v % NS) * kDbcRow + t] = tot;
        }
      }
      __syncthreads();
      // epilogue: add the wavefronts' partials; dx, ddelta, dz for 2 steps of one channel
      {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = eq * 2 + e;
          const int t = tb + i;
          const float* pr = s_red + er * kRedStride + i;
          float ys = pr[0], gds = pr[kChannelsPerGroup * kRedStride],
                gxsum = pr[2 * kChannelsPerGroup * kRedStride];
#pragma unroll
          for (int ww = 1; ww < NW; ++ww) {
            ys += pr[(ww * 3 + 0) * kChannelsPerGroup * kRedStride];
            gds += pr[(ww * 3 + 1) * kChannelsPerGroup * kRedStride];
            gxsum += pr[(ww * 3 + 2) * kChannelsPerGroup * kRedStride];
          }
          const f32x4 in = s_in[er * kInStride + in_col(t)];
          const float y = fmaf(eD, in.w, ys);
          const float vz = in.y * y;
          const float vx = fmaf(in.z, eD, gxsum);
          const float vd = gds * (p.softplus ? sigmoid_from_softplus(in.x) : 1.0f);
          dD_acc = fmaf(in.z, in.w, dD_acc);
          // (a padding step past L adds nothing: its vd is not zero when a final-state
          // gradient flows through it and delta takes no softplus)
          if (t < lt_len) dbias_acc += vd;
          // the step's inputs are dead now (this thread read them last): the slot holds the
          // outputs until the tile is written out
          s_in[er * kInStride + in_col(t)] = f32x4{vx, vd, vz, 0.0f};
        }
      }
      __syncthreads();  // s_red is reused by the next sub-tile
    }

    // the tile's outputs into registers (each thread reads the s_in slots of its own prologue
    // item, which only it overwrites next; s_dbc is written again after the next barrier)
    gather_outputs();
    if (!PREFETCH && tile > 0) issue(tile - 1, false);
  }
  put_outputs(0);

  // ---- per-workgroup partials of the batch-summed gradients, and dh0
  if (live) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (n0 + j >= p.N) continue;
      q.dA_part[(b * p.dim + d) * p.N + n0 + j] = da[j];
      if (q.dh0) q.dh0[(b * p.dim + d) * p.N + n0 + j] = gh[j];
    }
  }
  // the channel's four step groups, one per wavefront, added as (0 + 1) + (2 + 3)
  __syncthreads();  // every wavefront is past its last reads of s_red
  s_red[eq * 64 + er] = dD_acc;
  s_red[(4 + eq) * 64 + er] = dbias_acc;
  __syncthreads();
  if (elive && eq == 0) {
    q.dD_part[b * p.dim + ed] = (s_red[er] + s_red[64 + er]) + (s_red[128 + er] + s_red[192 + er]);
    q.dbias_part[b * p.dim + ed] =
        (s_red[256 + er] + s_red[320 + er]) + (s_red[384 + er] + s_red[448 + er]);
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
  // where the forward's planner takes 64-channel workgroups, narrow_one_pass: then the
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
    if (!narrow_one_pass(groups)) {
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
