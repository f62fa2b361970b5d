// gfx950 backward kernel (templates; instantiated per io dtype in scan_bwd_wide_{bf16,f32}.hip)
// for the cases the four-state kernel of scan_bwd.hip does not take:
// one A per head, dstate above 16 (up to 128), and the zero-order-hold rule.
//
// The layout is that of the other kernels: one workgroup = 64 channels of one batch entry,
// lane = channel, and NW wavefronts split the states (wavefront w owns states w*NS .. +NS).
// The states are recomputed from the checkpoints that the forward kernel's checkpoint pass
// stores every 8 steps (page "NL-345", §1 "Hardware-aware Algorithm": recomputation instead of
// stored states). A lane holds NS states, so an 8-step interval is processed in register
// blocks of SUB steps, last first: each block recomputes its start state from the checkpoint,
// then its SUB states, then runs the reverse recurrence over them. With one decay per head the
// exp (and the zero-order-hold ratio) is formed once per step and shared by all states.
//
// Gradients per step t, state n, with gh = dL/dh_t (gy = dL/dy before the gate):
//   gh += gy C_n;  dC_n += gy h_n;  gh_n carries dA_n back to step t-1
//   delta*B rule:  dB_n += gh delta x;  dx += gh delta B_n;  ddelta += gh (a dA h_prev + B x);
//                  da_n += gh dA h_prev delta
//   zero-order hold, B_bar = (dA - 1) / a B = delta g(w) B with w = delta a, g = expm1(w) / w:
//                  dB_n += gh delta g x;  dx += gh delta g B_n;  ddelta += gh (a dA h_prev + dA B x);
//                  da_n += gh (dA h_prev delta + delta^2 g'(w) B x)
// The sums over states go across wavefronts through LDS; the sums over channels of dB and dC
// are made over the wavefront's lanes through a wave-private LDS transpose and written as one
// partial per workgroup, which bwd_reduce_bc adds in a fixed order. In head mode the per-channel
// ddelta is summed over the channels of a head (a fixed-order reduction after this kernel),
// and so are dA and the bias gradient. Every reduction has a fixed order: results are
// deterministic.
#pragma once
#include "scan_bwd_common.h"

namespace ssm {
namespace wide {
constexpr int kT = 16;          // steps per tile (one load of the per-step inputs)
constexpr int kInS = kT + 1;    // entries per channel row of the per-step LDS arrays
constexpr int kSumS = 64 + 4;   // floats per column of the lane-sum scratch
constexpr int kHeadChunk = kHeadDeltaChunk;  // steps per workgroup of the head-mode delta reduction
constexpr int kDbcS = kT + 1;   // floats per (tensor, state) row of the tile's dB / dC partials
static_assert(kT % kCkptStep == 0, "a tile holds whole checkpoint intervals");
}  // namespace wide

// delta^2 g'(w) for w = delta a, g(w) = expm1(w) / w: g'(w) = (e^w - g) / w for |w| >= 1/2
// (e^w - g >= 0.2 there, so the roundings of dA = e^w and g cost a few 1e-7 relative), else the
// series 1/2 + w/3 + w^2/8 + w^3/30 + w^4/144 + w^5/840 + w^6/5760 + w^7/45360 (the first
// dropped term is below 3e-8 relative at |w| = 1/2).
__device__ __forceinline__ float zoh_dgdw_delta2(float dl, float w, float dA, float g) {
  float s = fmaf(w, 1.0f / 45360.0f, 1.0f / 5760.0f);
  s = fmaf(w, s, 1.0f / 840.0f);
  s = fmaf(w, s, 1.0f / 144.0f);
  s = fmaf(w, s, 1.0f / 30.0f);
  s = fmaf(w, s, 0.125f);
  s = fmaf(w, s, 1.0f / 3.0f);
  s = fmaf(w, s, 0.5f);
  const float closed = (dA - g) * __builtin_amdgcn_rcpf(w);
  return dl * dl * (fabsf(w) < 0.5f ? s : closed);
}

template <typename IO, int NS, int NW, int SUB, bool HEAD, bool ZOH, bool GATE>
__global__ void __launch_bounds__(64 * NW, 1) bwd_wide_kernel(const BwdParams q) {
  using namespace wide;
  constexpr int NT = 64 * NW;
  constexpr int NP = NS * NW;
  constexpr int V = IoTraits<IO>::kVec;
  constexpr int CPT = kT / V;                  // 16-byte chunks per channel row of a tile
  constexpr int ITEMS = kChannelsPerGroup * CPT;
  constexpr int NV = 2 * NS;                   // dC then dB of the lane's states at one step
  constexpr int NMB = kCkptStep / SUB;         // register blocks per checkpoint interval
  constexpr int RED = SUB + 1;
  constexpr int EITEMS = kChannelsPerGroup * SUB;
  constexpr int IPE = (EITEMS + NT - 1) / NT;  // epilogue items per thread
  static_assert(kCkptStep % SUB == 0, "register blocks tile the checkpoint interval");
  static_assert(64 % NV == 0 && NV % 4 == 0, "lane-sum layout");

  __shared__ __align__(16) f32x4 s_in[kChannelsPerGroup * kInS];  // delta, u = delta x, gy, x
  __shared__ float s_gz[GATE ? kChannelsPerGroup * kInS : 1];     // dy silu'(z)
  // B and C step-major: a wavefront's NS states of one step are NS consecutive floats, read as
  // NS / 4 16-byte words at one (wave-uniform) address each
  // (steps kBCRow floats apart, an odd multiple of 4: the fill's stores along the steps of a
  // state spread over 8 bank groups)
  constexpr int kBCRow = NP % 8 == 0 ? NP + 4 : NP;
  __shared__ __align__(16) float s_B[kT * kBCRow];
  __shared__ __align__(16) float s_C[kT * kBCRow];
  __shared__ float s_red[3 * NW * kChannelsPerGroup * RED];        // per-channel partial sums
  __shared__ __align__(16) float s_sum[NW * NV * kSumS];           // dB / dC lane sums
  // the tile's dC, dB partials (tensor, state, step), written out whole when the tile is done;
  // where that buffer would take the workgroup past 80 KB of LDS (two workgroups per CU with
  // four wavefronts), each step's sums are stored as they are made instead
  constexpr int kLdsRest = (int)(kChannelsPerGroup * kInS * sizeof(f32x4)) +
                           (GATE ? kChannelsPerGroup * kInS * 4 : 4) + 2 * kBCRow * kT * 4 +
                           3 * NW * kChannelsPerGroup * RED * 4 + NW * NV * kSumS * 4;
  constexpr bool kStageDbc = NW == 8 || kLdsRest + 2 * NP * kDbcS * 4 <= 80 * 1024;
  __shared__ float s_dbc[kStageDbc ? 2 * NP * kDbcS : 1];
  // head mode: each channel's ddelta (summed over the wavefronts) at the block's steps, for the
  // sums over runs of channels
  __shared__ float s_hd[HEAD ? kChannelsPerGroup * RED : 1];

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

  // ---- this lane's channel, its A and its gradient state
  const int64_t d = d0 + lane;
  const bool live = d < p.dim;
  // a * log2(e) for exp2 (sums weighted by a itself are formed with it and scaled by ln 2)
  float ap[HEAD ? 1 : NS];
  if constexpr (HEAD) {
    ap[0] = live ? p.A[d / p.headdim] * kLog2e : 0.0f;
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      ap[j] = (live && n0 + j < p.N) ? p.A[d * p.N + n0 + j] * kLog2e : 0.0f;
  }
  float gh[NS], da[HEAD ? 1 : NS];
#pragma unroll
  for (int j = 0; j < NS; ++j)
    gh[j] = (q.dhfin && live && n0 + j < p.N) ? q.dhfin[(b * p.dim + d) * p.N + n0 + j] : 0.0f;
#pragma unroll
  for (int j = 0; j < (HEAD ? 1 : NS); ++j) da[j] = 0.0f;

  float dD_acc[IPE], dbias_acc[IPE], eD_item[IPE];
#pragma unroll
  for (int r = 0; r < IPE; ++r) {
    dD_acc[r] = dbias_acc[r] = 0.0f;
    // D of the epilogue item's channel, read once (inside the loops it would be read, and
    // waited for, every block: the loops' stores might alias it)
    const int64_t ed = d0 + (tid + r * NT) / SUB;
    eD_item[r] = (ed < p.dim && p.D) ? p.D[min(ed, p.dim - 1)] : 0.0f;
  }

  float* const red = s_sum + w * NV * kSumS + lane;  // this lane's column entries
  const int rows_per_wg = kChannelsPerGroup / (HEAD ? (int)q.span : 1);

  for (int64_t tile = (L + kT - 1) / kT - 1; tile >= 0; --tile) {
    const int64_t t0 = tile * kT;
    const int len = (int)min<int64_t>(kT, L - t0);

    // ---- prologue: per (channel, step) values of the tile; padding steps are zero
    for (int item = tid; item < ITEMS; item += NT) {
      const int r = item / CPT, tl = (item % CPT) * V;
      const int64_t dd = d0 + r;
      const int64_t dv = min(dd, p.dim - 1);
      const int64_t drow = HEAD ? dv / p.headdim : dv;
      const int cnt = dd < p.dim ? max(0, min(V, len - tl)) : 0;
      float xv[V], dr[V], zv[V], gv[V];
      load_chunk<IO, true>(X + b * p.x_sb + dv * p.x_sd, t0 + tl, cnt, vec, xv);
      load_chunk<IO, true>(DL + b * p.dl_sb + drow * p.dl_sd, t0 + tl, cnt, vec, dr);
      load_chunk<IO, true>(DY + b * p.y_sb + dv * p.y_sd, t0 + tl, cnt, vec, gv);
      if constexpr (GATE) load_chunk<IO, true>(Z + b * p.z_sb + dv * p.z_sd, t0 + tl, cnt, vec, zv);
      const float bias = (dd < p.dim && p.delta_bias) ? p.delta_bias[drow] : 0.0f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float dl = 0.0f, u = 0.0f, gy = 0.0f, xx = 0.0f, gzf = 0.0f;
        if (e < cnt) {
          const float v = dr[e] + bias;
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
        s_in[r * kInS + tl + e] = f32x4{dl, u, gy, xx};
        if constexpr (GATE) s_gz[r * kInS + tl + e] = gzf;
      }
    }
    for (int i = tid; i < NP * kT; i += NT) {
      const int n = i / kT, t = i % kT;
      const bool on = n < p.N && t < len;
      s_B[t * kBCRow + n] = on ? to_f32(Bg[n * p.B_sn + t0 + t]) : 0.0f;
      s_C[t * kBCRow + n] = on ? to_f32(Cg[n * p.C_sn + t0 + t]) : 0.0f;
    }
    __syncthreads();

    // ---- checkpoint intervals of the tile, last first (one past L has no steps: skipped by
    // the whole workgroup alike)
#pragma unroll 1
    for (int k = kT / kCkptStep - 1; k >= 0; --k) {
      const int tb = k * kCkptStep;
      if (t0 + tb >= L) continue;
      const int64_t ci = tile * (kT / kCkptStep) + k;
      const float* const ck = p.ckpt + ((b * p.ntiles + ci) * p.N + n0) * p.dim + (live ? d : 0);

      // the wavefront's NS values of B or C at tile step t
      auto states_at = [&](const float* s, int t, float (&v)[NS]) __attribute__((always_inline)) {
        const f32x4* src = reinterpret_cast<const f32x4*>(s + t * kBCRow + n0);
#pragma unroll
        for (int k = 0; k < NS / 4; ++k) {
          const f32x4 w4 = src[k];
          v[4 * k] = w4.x; v[4 * k + 1] = w4.y; v[4 * k + 2] = w4.z; v[4 * k + 3] = w4.w;
        }
      };
      // one forward step of the recurrence at tile step t: h <- dA h + B_bar x
      auto fwd_step = [&](float (&hv)[NS], int t) __attribute__((always_inline)) {
        const f32x4 in = s_in[lane * kInS + t];
        float Bt[NS];
        states_at(s_B, t, Bt);
        float dAh = 1.0f, gH = 1.0f;
        if constexpr (HEAD) {
          dAh = __builtin_amdgcn_exp2f(in.x * ap[0]);
          if constexpr (ZOH) gH = zoh_ratio(dAh, in.x * ap[0]);
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          float dA, ub = in.y * Bt[j];
          if constexpr (HEAD) {
            dA = dAh;
            if constexpr (ZOH) ub *= gH;
          } else {
            dA = __builtin_amdgcn_exp2f(in.x * ap[j]);
            if constexpr (ZOH) ub *= zoh_ratio(dA, in.x * ap[j]);
          }
          hv[j] = fmaf(dA, hv[j], ub);
        }
      };

#pragma unroll 1
      for (int m = NMB - 1; m >= 0; --m) {
        const int tm = tb + m * SUB;  // first step of the block within the tile
        // the block's start state, from the interval's checkpoint (read again for every block:
        // registers are scarcer than the cached reads)
        float hs[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) hs[j] = (live && n0 + j < p.N) ? ck[j * p.dim] : 0.0f;
#pragma unroll 1
        for (int i = 0; i < m * SUB; ++i) fwd_step(hs, tb + i);
        // the block's states after each step (and the readout that dz needs)
        float hh[SUB][NS];
        float yp[SUB];
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
#pragma unroll
          for (int j = 0; j < NS; ++j) hh[i][j] = i == 0 ? hs[j] : hh[i - 1][j];
          fwd_step(hh[i], tm + i);
          float acc = 0.0f;
          if constexpr (GATE) {
            float Ct[NS];
            states_at(s_C, tm + i, Ct);
#pragma unroll
            for (int j = 0; j < NS; ++j) acc = fmaf(Ct[j], hh[i][j], acc);
          }
          yp[i] = acc;
        }
        // reverse recurrence over the block
        float* const ry = s_red + ((0 * NW + w) * kChannelsPerGroup + lane) * RED;
        float* const rg = s_red + ((1 * NW + w) * kChannelsPerGroup + lane) * RED;
        float* const rx = s_red + ((2 * NW + w) * kChannelsPerGroup + lane) * RED;
#pragma unroll
        for (int i = SUB - 1; i >= 0; --i) {
          const int t = tm + i;
          const f32x4 in = s_in[lane * kInS + t];
          const float dl = in.x, u = in.y, gy = in.z, xx = in.w;
          float dAh = 1.0f, gH = 1.0f;
          if constexpr (HEAD) {
            dAh = __builtin_amdgcn_exp2f(dl * ap[0]);
            if constexpr (ZOH) gH = zoh_ratio(dAh, dl * ap[0]);
          }
          float gd = 0.0f, sb = 0.0f, sbA = 0.0f, s1 = 0.0f;
          float Bt[NS], Ct[NS];
          states_at(s_B, t, Bt);
          states_at(s_C, t, Ct);
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const float Bv = Bt[j];
            const float Cv = Ct[j];
            gh[j] = fmaf(gy, Cv, gh[j]);
            red[j * kSumS] = gy * hh[i][j];  // dC
            const float hp = i == 0 ? hs[j] : hh[i - 1][j];
            float dA, dBv;
            if constexpr (HEAD) {
              dA = dAh;
              s1 = fmaf(gh[j], hp, s1);
              dBv = gh[j] * (ZOH ? u * gH : u);
              sb = fmaf(gh[j], Bv, sb);
            } else {
              dA = __builtin_amdgcn_exp2f(dl * ap[j]);
              const float gt = gh[j] * (hp * dA);
              gd = fmaf(gt, ap[j], gd);  // times ln 2 below: sum of gt * a
              da[j] = fmaf(gt, dl, da[j]);
              if constexpr (ZOH) {
                const float w2 = dl * ap[j] * kLn2;
                const float g = zoh_ratio(dA, dl * ap[j]);
                dBv = gh[j] * (u * g);
                sb = fmaf(gh[j], Bv * g, sb);     // for dx
                sbA = fmaf(gh[j], Bv * dA, sbA);  // for ddelta
                da[j] = fmaf(gh[j] * Bv, xx * zoh_dgdw_delta2(dl, w2, dA, g), da[j]);
              } else {
                dBv = gh[j] * u;
                sb = fmaf(gh[j], Bv, sb);
              }
            }
            red[(NS + j) * kSumS] = dBv;  // dB
            gh[j] *= dA;
          }
          float gdel, gxp;
          if constexpr (HEAD) {
            gd = ap[0] * kLn2 * dAh * s1;
            da[0] = fmaf(dl * dAh, s1, da[0]);
            if constexpr (ZOH) {
              const float qz = zoh_dgdw_delta2(dl, dl * ap[0] * kLn2, dAh, gH);
              da[0] = fmaf(qz * xx, sb, da[0]);
              gdel = fmaf(xx * dAh, sb, gd);
              gxp = dl * gH * sb;
            } else {
              gdel = fmaf(xx, sb, gd);
              gxp = dl * sb;
            }
          } else if constexpr (ZOH) {
            gdel = fmaf(xx, sbA, gd * kLn2);
            gxp = dl * sb;
          } else {
            gdel = fmaf(xx, sb, gd * kLn2);
            gxp = dl * sb;
          }
          ry[i] = yp[i];
          rg[i] = gdel;
          rx[i] = gxp;
          // sum this step's dC, dB over the wavefront's lanes (channels): lane sums value
          // col = lane % NV over lanes part * NV .. + NV, then the 64 / NV parts combine
          wave_lds_sync();
          {
            const int col = lane % NV, part = lane / NV;
            const f32x4* src =
                reinterpret_cast<const f32x4*>(s_sum + (w * NV + col) * kSumS + part * NV);
            f32x4 acc4 = src[0];
#pragma unroll
            for (int r4 = 1; r4 < NV / 4; ++r4) acc4 += src[r4];
            float sum = (acc4.x + acc4.y) + (acc4.z + acc4.w);
#pragma unroll
            for (int off = NV; off < 64; off <<= 1) sum = xor_sum(sum, off);
            if constexpr (kStageDbc) {
              // into the tile buffer (rows of padding states and steps past L are never written
              // out)
              if (lane < NV) s_dbc[((col < NS ? 0 : NP) + n0 + col % NS) * kDbcS + t] = sum;
            } else {
              const int j = col % NS;
              const int64_t tt = t0 + t;
              if (lane < NV && n0 + j < p.N && tt < L) {
                float* dst = col < NS ? q.dC_part : q.dB_part;
                dst[((b * p.groups_per_batch + wg) * p.N + n0 + j) * L + tt] = sum;
              }
            }
          }
          wave_lds_sync();
        }
        __syncthreads();

        // ---- epilogue: add the wavefronts' partials; dx, dz (and ddelta per channel)
#pragma unroll
        for (int r = 0; r < IPE; ++r) {
          const int item = tid + r * NT;
          if (EITEMS % NT != 0 && item >= EITEMS) continue;
          const int er = item / SUB, i = item % SUB;
          const int t = tm + i;
          const int64_t ed = d0 + er, tt = t0 + t;
          float ys = 0.0f, gds = 0.0f, gxs = 0.0f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) {
            ys += s_red[((0 * NW + ww) * kChannelsPerGroup + er) * RED + i];
            gds += s_red[((1 * NW + ww) * kChannelsPerGroup + er) * RED + i];
            gxs += s_red[((2 * NW + ww) * kChannelsPerGroup + er) * RED + i];
          }
          const f32x4 in = s_in[er * kInS + t];
          const float eD = eD_item[r];
          const float vx = fmaf(in.z, eD, gxs);
          dD_acc[r] = fmaf(in.z, in.w, dD_acc[r]);
          float vz = 0.0f, vd = 0.0f;
          if constexpr (GATE) vz = s_gz[er * kInS + t] * fmaf(eD, in.w, ys);
          if constexpr (HEAD) {
            s_hd[er * RED + i] = gds;
          } else {
            vd = gds * (p.softplus ? sigmoid_from_softplus(in.x) : 1.0f);
            // (a padding step past L adds nothing: its vd is not zero when a final-state
            // gradient flows through it and delta takes no softplus)
            if (ed < p.dim && tt < L) dbias_acc[r] += vd;
          }
          // the step's inputs are dead now (later blocks take earlier steps): the slot holds
          // the outputs until the tile is written out
          s_in[er * kInS + t] = f32x4{vx, vd, vz, 0.0f};
        }
        __syncthreads();  // s_red is reused by the next block; s_hd is complete
        if constexpr (HEAD) {
          // ddelta before the activation, summed over each run of `span` channels (all in one
          // head; the head's rows are added by bwd_head_delta). A wavefront takes 64 / span
          // (run, step) items at once, a lane per channel, and adds each run's lanes by lane
          // exchanges in a fixed order.
          const int span = (int)q.span;  // a power of two, at most 64
          const int per = 64 / span;
          const int nitems = rows_per_wg * SUB;
          const int g = lane / span, c = lane % span;
          for (int base = w * per; base < nitems; base += NW * per) {
            const int item = base + g;
            const int rr = item / SUB, i = item % SUB;
            float v = item < nitems ? s_hd[(rr * span + c) * RED + i] : 0.0f;
            for (int off = 1; off < span; off <<= 1) v = xor_sum(v, off);
            const int64_t tt = t0 + tm + i;
            if (c == 0 && item < nitems && d0 + (int64_t)rr * span < p.dim && tt < L)
              q.ddl_part[(b * (p.dim / span) + d0 / span + rr) * L + tt] = v;
          }
        }
      }
    }
    // the tile's dC, dB partials: whole rows of its steps (16-byte stores where the rows allow
    // them). Every step's sums are in s_dbc (the last block ended with a barrier).
    if constexpr (kStageDbc) {
      constexpr int Q4 = kT / 4;
      for (int item = tid; item < 2 * NP * Q4; item += NT) {
        const int row = item / Q4, t4 = 4 * (item % Q4);
        const int n = row % NP;
        if (n >= p.N || t4 >= len) continue;
        float* dst = (row < NP ? q.dC_part : q.dB_part) +
                     ((b * p.groups_per_batch + wg) * p.N + n) * L + t0 + t4;
        const float* src = s_dbc + row * kDbcS + t4;
        if (q.part_vec && t4 + 4 <= len) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{src[0], src[1], src[2], src[3]};
        } else {
          for (int e = 0; e < 4 && t4 + e < len; ++e) dst[e] = src[e];
        }
      }
    }
    // dx, dz (and ddelta per channel) of the tile from the s_in slots, 16 bytes per store, by
    // the thread whose prologue item covers the same slots (its next prologue writes them)
    for (int item = tid; item < ITEMS; item += NT) {
      const int r = item / CPT, tl = (item % CPT) * V;
      const int64_t dd = d0 + r;
      const int cnt = dd < p.dim ? max(0, min(V, len - tl)) : 0;
      if (cnt == 0) continue;
      float vx[V], vd[V], vz[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const f32x4 o = s_in[r * kInS + tl + e];
        vx[e] = o.x;
        vd[e] = o.y;
        vz[e] = o.z;
      }
      const bool full = q.vec_out != 0;
      store_chunk<IO>(static_cast<IO*>(q.dx) + b * p.x_sb + dd * p.x_sd, t0 + tl, cnt, full, vx);
      if constexpr (GATE)
        store_chunk<IO>(static_cast<IO*>(q.dz) + b * p.z_sb + dd * p.z_sd, t0 + tl, cnt, full, vz);
      if constexpr (!HEAD)
        store_chunk<IO>(static_cast<IO*>(q.ddelta) + b * p.dl_sb + dd * p.dl_sd, t0 + tl, cnt,
                        full, vd);
    }
    // the next tile's prologue overwrites s_in, s_B, s_C and its steps s_dbc: every wavefront is
    // past its reads (the barrier that begins the next tile's steps)
  }

  // ---- per-workgroup partials of the batch-summed gradients, and dh0
  if (live) {
    if constexpr (HEAD) {
      if (n0 < p.N) q.dA_part[(b * p.dim + d) * p.N + n0] = da[0];
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (n0 + j < p.N) q.dA_part[(b * p.dim + d) * p.N + n0 + j] = da[j];
    }
    if (q.dh0) {
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (n0 + j < p.N) q.dh0[(b * p.dim + d) * p.N + n0 + j] = gh[j];
    }
  }
  // dD (and dbias per channel): sum over the SUB consecutive lanes that hold a channel's steps
#pragma unroll
  for (int r = 0; r < IPE; ++r) {
    float sd = dD_acc[r], sbias = dbias_acc[r];
#pragma unroll
    for (int off = 1; off < SUB; off <<= 1) {
      sd += __shfl_xor(sd, off);
      sbias += __shfl_xor(sbias, off);
    }
    const int item = tid + r * NT;
    const int64_t ed = d0 + item / SUB;
    if ((EITEMS % NT == 0 || item < EITEMS) && item % SUB == 0 && ed < p.dim) {
      q.dD_part[b * p.dim + ed] = sd;
      if constexpr (!HEAD) q.dbias_part[b * p.dim + ed] = sbias;
    }
  }
}

// Head mode: ddelta[b, h, t] = act'(v) * (sum of the head's channel partials), and the partial
// sums of ddelta over each chunk of kHeadChunk steps for the bias gradient. One workgroup per
// (head, batch entry, chunk); fixed-order sums.
template <typename IO>
__global__ void __launch_bounds__(256) bwd_head_delta(const BwdParams q) {
  using namespace wide;
  const ScanParams& p = q.f;
  const int64_t nheads = p.dim / p.headdim;
  const int64_t nchunks = (p.L + kHeadChunk - 1) / kHeadChunk;
  const int64_t chunk = blockIdx.x % nchunks;
  const int64_t b = (blockIdx.x / nchunks) % p.batch;
  const int64_t h = blockIdx.x / (nchunks * p.batch);
  const int64_t span = q.span, rows = p.dim / span, rph = p.headdim / span;
  const float bias = p.delta_bias ? p.delta_bias[h] : 0.0f;
  const IO* DL = static_cast<const IO*>(p.delta) + b * p.dl_sb + h * p.dl_sd;
  IO* DDL = static_cast<IO*>(q.ddelta) + b * p.dl_sb + h * p.dl_sd;
  constexpr int kPer = kHeadChunk / 256;
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int64_t t = chunk * kHeadChunk + e * 256 + threadIdx.x;
    if (t >= p.L) continue;
    float s = 0.0f;
    for (int64_t r = 0; r < rph; ++r) s += q.ddl_part[(b * rows + h * rph + r) * p.L + t];
    float f = 1.0f;
    if (p.softplus) {
      const float v = to_f32(DL[t]) + bias;
      f = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));  // sigmoid(v)
    }
    const float g = s * f;
    store_elem(DDL + t, g);
    acc += g;
  }
  __shared__ float s_acc[256];
  s_acc[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) s_acc[threadIdx.x] += s_acc[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) q.dbias_hpart[(h * p.batch + b) * nchunks + chunk] = s_acc[0];
  (void)nheads;
}

// The checkpoint pass (the forward kernel in its checkpoint mode: the state before every 8th
// step) for the cases this kernel takes; the state split of the forward kernel does not change
// the checkpoints' layout.
template <typename IO, int NS4, bool HEAD, bool ZOH>
static hipError_t wide_ckpt(const BwdParams& q, hipStream_t stream) {
  const ScanParams& p = q.f;
  hipLaunchKernelGGL((scan_fwd_kernel<IO, NS4, kWavesPerGroup, HEAD, false, false, ZOH, true>),
                     dim3((unsigned)(p.batch * p.groups_per_batch), 1), dim3(64 * kWavesPerGroup),
                     0, stream, static_cast<const IO*>(p.x), static_cast<const IO*>(p.delta),
                     static_cast<const IO*>(p.B), static_cast<const IO*>(p.C),
                     static_cast<const IO*>(nullptr), static_cast<IO*>(nullptr), p.A, p.D,
                     p.delta_bias, nullptr, nullptr, p);
  return hipGetLastError();
}

template <typename IO, int NS, int NW, int SUB, bool HEAD, bool ZOH>
static hipError_t wide_cfg(const BwdParams& q, hipStream_t stream) {
  const ScanParams& p = q.f;
  constexpr int NS4 = NS * NW / kWavesPerGroup;  // the same padded state count in 4 wavefronts
  hipError_t e = wide_ckpt<IO, NS4, HEAD, ZOH>(q, stream);
  if (e != hipSuccess) return e;
  const unsigned groups = (unsigned)(p.batch * p.groups_per_batch);
  if (p.z)
    hipLaunchKernelGGL((bwd_wide_kernel<IO, NS, NW, SUB, HEAD, ZOH, true>), dim3(groups),
                       dim3(64 * NW), 0, stream, q);
  else
    hipLaunchKernelGGL((bwd_wide_kernel<IO, NS, NW, SUB, HEAD, ZOH, false>), dim3(groups),
                       dim3(64 * NW), 0, stream, q);
  return hipGetLastError();
}

template <typename IO, bool HEAD, bool ZOH>
static hipError_t wide_n(const BwdParams& q, hipStream_t stream) {
  const int64_t N = q.f.N;
  // register blocks: SUB x NS recomputed states per lane (one exp per state in diagonal mode
  // needs more registers than one per head)
  constexpr int SUB8 = HEAD ? 8 : 4, SUB16 = HEAD ? 4 : 2;
  if (N <= 16) return wide_cfg<IO, 4, 4, 8, HEAD, ZOH>(q, stream);
  if (N <= 32) return wide_cfg<IO, 8, 4, SUB8, HEAD, ZOH>(q, stream);
  if (N <= 64) return wide_cfg<IO, 16, 4, SUB16, HEAD, ZOH>(q, stream);
  return wide_cfg<IO, 16, 8, SUB16, HEAD, ZOH>(q, stream);  // N <= 128 (checked by the caller)
}

// Checkpoint pass, the reverse kernel and (head mode) the ddelta reduction; the caller then runs
// the dB / dC and parameter reductions.
template <typename IO>
static hipError_t wide_io(const BwdParams& q, hipStream_t stream) {
  const ScanParams& p = q.f;
  hipError_t e;
  if (q.head) e = p.zoh ? wide_n<IO, true, true>(q, stream) : wide_n<IO, true, false>(q, stream);
  else e = p.zoh ? wide_n<IO, false, true>(q, stream) : wide_n<IO, false, false>(q, stream);
  if (e != hipSuccess || !q.head) return e;
  const int64_t nchunks = (p.L + wide::kHeadChunk - 1) / wide::kHeadChunk;
  const int64_t nheads = p.dim / p.headdim;
  hipLaunchKernelGGL(bwd_head_delta<IO>, dim3((unsigned)(nheads * p.batch * nchunks)), dim3(256),
                     0, stream, q);
  return hipGetLastError();
}

}  // namespace ssm
