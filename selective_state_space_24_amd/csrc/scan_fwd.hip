// gfx950 kernels of the selective-scan forward pass.
//
// Work decomposition (one workgroup = 64 channels of one batch entry x one segment of L):
//   * lane l of every wavefront owns channel d0 + l; wavefront w owns states [w*NS, (w+1)*NS).
//     The state h (NS fp32 values per lane) lives in VGPRs for the whole segment and is never
//     written to memory (the pages' hardware-aware scan keeps the expanded state on chip).
//   * time advances in tiles of kTB steps. Per tile, a prologue (all threads) loads x, delta and
//     z with row-contiguous 16-byte loads, computes the step size delta = softplus(raw + bias)
//     and u = delta * x once per (channel, t), and stages those plus the tile of B and C
//     (shared by all channels of the group) in LDS as fp32.
//   * the recurrence sweeps the tile per lane. B_tn and C_tn are the same for every lane, so a
//     wavefront fetches 16 (state, step) values per VGPR (one per lane of a 16-lane row,
//     replicated over the four rows) and broadcasts each one with the DPP row_newbcast operand
//     modifier, which folds into the multiply that consumes it.
//   * each wavefront's partial readout sum_n C h over its states goes to LDS; an epilogue adds
//     the partials, the D skip and the silu(z) gate and stores y with 16-byte stores.
//   * a sequence split into segments along L (too few channels to fill the chip) first runs a
//     summary pass per segment: the final state from a zero start and the segment's sum of
//     delta, whose exp(A * sum) is the segment's decay. The output pass of segment s composes the
//     summaries of segments < s into its initial state. The pairs (decay, offset) compose
//     associatively, which is what makes the split exact up to rounding.
//
// Arithmetic: fp32 throughout. dA = 2^(delta * A * log2 e) with the hardware exp2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_internal.h"

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTB = 32;                 // time steps per tile
constexpr int kDuStride = 2 * kTB + 4;  // floats per channel row of (delta, u) in LDS
constexpr int kPartStride = kTB + 4;    // floats per channel row of partial readouts
constexpr int kBcStride = kTB + 4;      // floats per state row of the B / C tile

typedef uint16_t bf16_bits;
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename IO>
struct IoTraits;
template <>
struct IoTraits<float> {
  static constexpr int kVec = 4;  // elements per 16-byte access
};
template <>
struct IoTraits<bf16_bits> {
  static constexpr int kVec = 8;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_bits v) { return __uint_as_float((uint32_t)v << 16); }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const float2v f = {lo, hi};
  const bf16x2v h = __builtin_convertvector(f, bf16x2v);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(bf16_bits* p, float v) {
  *p = (bf16_bits)(pack_bf16x2(v, 0.0f) & 0xffffu);
}

template <bool STREAM>
__device__ __forceinline__ u32x4 load16(const void* ptr) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
  else return *reinterpret_cast<const u32x4*>(ptr);
}

// Loads row[t .. t+kVec) (cnt of them valid, the rest zero) as fp32. STREAM marks data read
// once (nontemporal hint); B and C rows are reused by every workgroup of a batch entry.
template <typename IO, bool STREAM>
__device__ __forceinline__ void load_chunk(const IO* __restrict__ row, int64_t t, int cnt,
                                           bool vec_ok, float (&out)[IoTraits<IO>::kVec]) {
  constexpr int V = IoTraits<IO>::kVec;
  if (vec_ok && cnt == V) {
    const u32x4 w = load16<STREAM>(row + t);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    if constexpr (V == 8) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[2 * k] = __uint_as_float(ws[k] << 16);
        out[2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = __uint_as_float(ws[k]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) out[e] = (e < cnt) ? to_f32(row[t + e]) : 0.0f;
  }
}

// The kVec io values of a 16-byte word as fp32.
template <typename IO>
__device__ __forceinline__ void unpack16(const u32x4 w, float (&out)[IoTraits<IO>::kVec]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  if constexpr (IoTraits<IO>::kVec == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[2 * k] = __uint_as_float(ws[k] << 16);
      out[2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = __uint_as_float(ws[k]);
  }
}

template <typename IO>
__device__ __forceinline__ void store_chunk(IO* __restrict__ row, int64_t t, int cnt, bool vec_ok,
                                            const float (&v)[IoTraits<IO>::kVec]) {
  constexpr int V = IoTraits<IO>::kVec;
  if (vec_ok && cnt == V) {
    uint32_t ws[4];
    if constexpr (V == 8) {
#pragma unroll
      for (int k = 0; k < 4; ++k) ws[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) ws[k] = __float_as_uint(v[k]);
    }
    const u32x4 q = {ws[0], ws[1], ws[2], ws[3]};
    __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(row + t));
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (e < cnt) store_elem(row + t + e, v[e]);
  }
}

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e), e = e^-|v| in (0, 1].
// log1p(e) = ln(u) + (e - (u - 1)) / u with u = fl(1 + e): the second term restores what the
// rounding of u lost; dividing it by u instead of 1 changes the result by at most one rounding
// of u times e/(1+e), so it is dropped. ln(u) uses the hardware log2 on u in [1, 2].
__device__ __forceinline__ float softplus_f32(float v) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
  const float u = 1.0f + e;
  const float corr = e - (u - 1.0f);
  return fmaxf(v, 0.0f) + fmaf(__builtin_amdgcn_logf(u), kLn2, corr);
}

// silu(z) = z * sigmoid(z), with the hardware exp2 and reciprocal
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Lane (16 * row + I)'s value of v, given to every lane of the row (DPP row_newbcast:I).
template <int I>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + I, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_bcast_k(float v, int i) {
  switch (i) {
    case 0: return row_bcast<0>(v);   case 1: return row_bcast<1>(v);
    case 2: return row_bcast<2>(v);   case 3: return row_bcast<3>(v);
    case 4: return row_bcast<4>(v);   case 5: return row_bcast<5>(v);
    case 6: return row_bcast<6>(v);   case 7: return row_bcast<7>(v);
    case 8: return row_bcast<8>(v);   case 9: return row_bcast<9>(v);
    case 10: return row_bcast<10>(v); case 11: return row_bcast<11>(v);
    case 12: return row_bcast<12>(v); case 13: return row_bcast<13>(v);
    case 14: return row_bcast<14>(v); default: return row_bcast<15>(v);
  }
}

// NS states per wavefront, NW wavefronts (N <= NS*NW); HEAD: one A and one delta per head;
// SUMMARY: the segment summary pass (no readout, no y).
template <typename IO, int NS, int NW, bool HEAD, bool SUMMARY>
__global__ void __launch_bounds__(64 * NW)
    scan_fwd_kernel(const IO* __restrict__ X, const IO* __restrict__ DL, const IO* __restrict__ Bm,
                    const IO* __restrict__ Cm, const IO* __restrict__ Z, IO* __restrict__ Y,
                    const float* __restrict__ Am, const float* __restrict__ Dm,
                    const float* __restrict__ bias_p, float* __restrict__ hend,
                    float* __restrict__ dsum, const ScanParams p) {
  static_assert(NS % 4 == 0, "states are swept in chunks of four");
  constexpr int NT = 64 * NW;
  constexpr int NP = NS * NW;  // padded state count
  constexpr int V = IoTraits<IO>::kVec;
  constexpr int CPR = kTB / V;  // 16-byte chunks per row of a tile
  constexpr int ITEMS = kChannelsPerGroup * CPR;
  constexpr int IPT = (ITEMS + NT - 1) / NT;
  constexpr int BC_ITEMS = NP * CPR;
  __shared__ __align__(16) float s_du[kChannelsPerGroup * kDuStride];
  __shared__ __align__(16) float s_B[NP * kBcStride];
  __shared__ __align__(16) float s_C[SUMMARY ? 4 : NP * kBcStride];
  __shared__ __align__(16) float s_part[SUMMARY ? 4 : NW * kChannelsPerGroup * kPartStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b = blockIdx.x / p.groups_per_batch;
  const int64_t d0 = (blockIdx.x % p.groups_per_batch) * kChannelsPerGroup;
  const int seg = blockIdx.y;
  const int64_t t_begin = (int64_t)seg * p.seg_len;
  const int64_t t_end = min(p.L, t_begin + p.seg_len);
  const bool vec_ok = p.vec_io != 0;
  const bool bc_vec = p.bc_vec != 0;
  const bool has_z = !SUMMARY && Z != nullptr;

  // B/C group of this workgroup's channels (the host guarantees one group per workgroup)
  const int64_t grp = d0 / (p.dim / p.ngroups);
  const IO* __restrict__ Bg = Bm + b * p.B_sb + grp * p.B_sg;
  const IO* __restrict__ Cg = Cm + b * p.C_sb + grp * p.C_sg;
  const int n0 = w * NS;

  // ---- per-lane constants of channel d = d0 + lane
  const int64_t d = d0 + lane;
  const bool live = d < p.dim;
  float ap[HEAD ? 1 : NS];
  if constexpr (HEAD) {
    ap[0] = live ? Am[d / p.headdim] * kLog2e : 0.0f;
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      ap[j] = (live && n0 + j < p.N) ? Am[d * p.N + n0 + j] * kLog2e : 0.0f;
  }

  float h[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) h[j] = 0.0f;
  if (!SUMMARY && seg > 0 && live) {
    // compose the summaries of segments 0 .. seg-1: h <- exp(A * sum delta) h + h_end
    const int64_t base = (b * p.dim + d) * p.nseg;
    for (int s = 0; s < seg; ++s) {
      const float ds = dsum[base + s];
      const float* he = hend + (base + s) * p.N;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float a;
        if constexpr (HEAD) a = ap[0]; else a = ap[j];
        if (n0 + j < p.N) h[j] = __builtin_amdgcn_exp2f(a * ds) * h[j] + he[n0 + j];
      }
    }
  }
  double dsum_total = 0.0;

  float xkeep[IPT][V];
  float zkeep[IPT][V];

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTB) {
    const int tb_len = (int)min<int64_t>(kTB, t_end - t0);

    // ---- prologue 1: delta and u = delta * x of the tile, into LDS. Steps past the end of the
    // sequence get delta = u = 0, which leaves h unchanged (dA = 1, dB x = 0).
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      if (ITEMS % NT == 0 || item < ITEMS) {
        const int r = item / CPR;
        const int tl = (item % CPR) * V;
        const int64_t dd = d0 + r;
        const int cnt = max(0, min(V, tb_len - tl));
        float xv[V], dv[V], zv[V];
        float bias = 0.0f;
        if (dd < p.dim && cnt > 0) {
          const int64_t drow = HEAD ? dd / p.headdim : dd;
          load_chunk<IO, true>(X + b * p.x_sb + dd * p.x_sd, t0 + tl, cnt, vec_ok, xv);
          load_chunk<IO, true>(DL + b * p.dl_sb + drow * p.dl_sd, t0 + tl, cnt, vec_ok, dv);
          if (has_z) load_chunk<IO, true>(Z + b * p.z_sb + dd * p.z_sd, t0 + tl, cnt, vec_ok, zv);
          if (bias_p) bias = bias_p[drow];
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) { xv[e] = 0.0f; dv[e] = 0.0f; zv[e] = 0.0f; }
        }
        float du[2 * V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float v = dv[e] + bias;
          const float dl = (e < cnt) ? (p.softplus ? softplus_f32(v) : v) : 0.0f;
          du[2 * e] = dl;
          du[2 * e + 1] = dl * xv[e];
          xkeep[it][e] = xv[e];
          zkeep[it][e] = has_z ? zv[e] : 0.0f;
        }
        float4* dst = reinterpret_cast<float4*>(&s_du[r * kDuStride + 2 * tl]);
#pragma unroll
        for (int k = 0; k < V / 2; ++k)
          dst[k] = make_float4(du[4 * k], du[4 * k + 1], du[4 * k + 2], du[4 * k + 3]);
      }
    }
    // ---- prologue 2: the B (and C) tile as fp32; padded states and steps are zero
    for (int item = tid; item < BC_ITEMS; item += NT) {
      const int n = item / CPR;
      const int tl = (item % CPR) * V;
      const int cnt = max(0, min(V, tb_len - tl));
      float bv[V], cv[V];
      if (n < p.N && cnt > 0) {
        load_chunk<IO, false>(Bg + (int64_t)n * p.B_sn, t0 + tl, cnt, bc_vec, bv);
        if (!SUMMARY) load_chunk<IO, false>(Cg + (int64_t)n * p.C_sn, t0 + tl, cnt, bc_vec, cv);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) { bv[e] = 0.0f; cv[e] = 0.0f; }
      }
      float4* db = reinterpret_cast<float4*>(&s_B[n * kBcStride + tl]);
#pragma unroll
      for (int k = 0; k < V / 4; ++k)
        db[k] = make_float4(bv[4 * k], bv[4 * k + 1], bv[4 * k + 2], bv[4 * k + 3]);
      if constexpr (!SUMMARY) {
        float4* dc = reinterpret_cast<float4*>(&s_C[n * kBcStride + tl]);
#pragma unroll
        for (int k = 0; k < V / 4; ++k)
          dc[k] = make_float4(cv[4 * k], cv[4 * k + 1], cv[4 * k + 2], cv[4 * k + 3]);
      }
    }
    __syncthreads();

    // ---- recurrence over the tile: lane = channel, this wavefront's NS states
    const int ri = lane & 15;  // slot in a 16-lane row: state ri / 4, step ri % 4
    for (int tt = 0; tt < tb_len; tt += 8) {
      float dl[8], u[8];
      const float4* src = reinterpret_cast<const float4*>(&s_du[lane * kDuStride + 2 * tt]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = src[k];
        dl[2 * k] = q.x; u[2 * k] = q.y; dl[2 * k + 1] = q.z; u[2 * k + 1] = q.w;
      }
      float acc[8];
      float dA_head[HEAD ? 8 : 1];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[k] = 0.0f;
        if constexpr (HEAD) dA_head[k] = __builtin_amdgcn_exp2f(dl[k] * ap[0]);
      }
      if constexpr (SUMMARY) {
        float s8 = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s8 += dl[k];
        dsum_total += (double)s8;
      }
#pragma unroll
      for (int jc = 0; jc < NS; jc += 4) {
        // 16 (state, step) values per register: states n0+jc .. +3 and steps tt .. tt+3 (lo),
        // tt+4 .. tt+7 (hi)
        const int bc_off = (n0 + jc + (ri >> 2)) * kBcStride + tt + (ri & 3);
        const float b_lo = s_B[bc_off], b_hi = s_B[bc_off + 4];
        float c_lo = 0.0f, c_hi = 0.0f;
        if constexpr (!SUMMARY) { c_lo = s_C[bc_off]; c_hi = s_C[bc_off + 4]; }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int slot = j * 4 + (k & 3);
            float dA;
            if constexpr (HEAD) dA = dA_head[k]; else dA = __builtin_amdgcn_exp2f(dl[k] * ap[jc + j]);
            const float bb = row_bcast_k(k < 4 ? b_lo : b_hi, slot);
            h[jc + j] = fmaf(dA, h[jc + j], u[k] * bb);
            if constexpr (!SUMMARY) {
              const float cc = row_bcast_k(k < 4 ? c_lo : c_hi, slot);
              acc[k] = fmaf(cc, h[jc + j], acc[k]);
            }
          }
        }
      }
      if constexpr (!SUMMARY) {
        float4* dst = reinterpret_cast<float4*>(&s_part[(w * kChannelsPerGroup + lane) * kPartStride + tt]);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      }
    }
    __syncthreads();

    // ---- epilogue: y = (sum of partial readouts + D x) * silu(z)
    if constexpr (!SUMMARY) {
#pragma unroll
      for (int it = 0; it < IPT; ++it) {
        const int item = tid + it * NT;
        if (ITEMS % NT == 0 || item < ITEMS) {
          const int r = item / CPR;
          const int tl = (item % CPR) * V;
          const int64_t dd = d0 + r;
          const int cnt = max(0, min(V, tb_len - tl));
          if (dd < p.dim && cnt > 0) {
            const float Dd = Dm ? Dm[dd] : 0.0f;
            float yv[V];
#pragma unroll
            for (int e4 = 0; e4 < V; e4 += 4) {
              float4 s4 = *reinterpret_cast<const float4*>(&s_part[r * kPartStride + tl + e4]);
#pragma unroll
              for (int ww = 1; ww < NW; ++ww) {
                const float4 q = *reinterpret_cast<const float4*>(
                    &s_part[(ww * kChannelsPerGroup + r) * kPartStride + tl + e4]);
                s4.x += q.x; s4.y += q.y; s4.z += q.z; s4.w += q.w;
              }
              yv[e4] = s4.x; yv[e4 + 1] = s4.y; yv[e4 + 2] = s4.z; yv[e4 + 3] = s4.w;
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
              float yy = fmaf(Dd, xkeep[it][e], yv[e]);
              if (has_z) yy *= silu_f32(zkeep[it][e]);
              yv[e] = yy;
            }
            store_chunk<IO>(Y + b * p.y_sb + dd * p.y_sd, t0 + tl, cnt, vec_ok, yv);
          }
        }
      }
    }
  }

  if constexpr (SUMMARY) {
    if (live) {
      const int64_t base = (b * p.dim + d) * p.nseg + seg;
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (n0 + j < p.N) hend[base * p.N + n0 + j] = h[j];
      if (w == 0) dsum[base] = (float)dsum_total;
    }
  }
}

// Sum of v over the four 16-lane rows, transposed over four steps: on return, row r of the
// result holds the row-sum of p[r] (per lane position within the row). gfx950's
// v_permlane32_swap exchanges the upper half of its first operand with the lower half of its
// second; v_permlane16_swap exchanges the odd rows of the first with the even rows of the second.
__device__ __forceinline__ float rows_transpose_sum4(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows: p0(0+2) p0(1+3) p2(0+2) p2(1+3)
  const float s13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// One wavefront per workgroup: 16 channels x 4 rows. Lane (row, ci) owns channel d0 + ci and the
// states [row*NS, row*NS + NS); the readout over the four rows is summed with cross-row lane
// swaps, so wavefronts never wait for each other. Global loads of the next tile are issued as
// soon as the current tile's raw registers have been consumed, and complete while the
// recurrence runs.
template <typename IO, int NS, bool HEAD, bool SUMMARY>
__global__ void __launch_bounds__(64)
    scan_rows_kernel(const IO* __restrict__ X, const IO* __restrict__ DL, const IO* __restrict__ Bm,
                     const IO* __restrict__ Cm, const IO* __restrict__ Z, IO* __restrict__ Y,
                     const float* __restrict__ Am, const float* __restrict__ Dm,
                     const float* __restrict__ bias_p, float* __restrict__ hend,
                     float* __restrict__ dsum, const ScanParams p) {
  static_assert(NS % 4 == 0, "states are swept in chunks of four");
  constexpr int CH = 16;       // channels per wavefront
  constexpr int NP = 4 * NS;   // padded state count
  constexpr int V = IoTraits<IO>::kVec;
  constexpr int CPR = kTB / V;  // 16-byte chunks per row of a tile
  constexpr int IPT = CH * CPR / 64;
  constexpr int BPT = NP * CPR / 64;
  static_assert(IPT >= 1 && BPT >= 1 && CH * CPR % 64 == 0 && NP * CPR % 64 == 0, "tile shape");
  __shared__ __align__(16) float s_du[CH * kDuStride];
  __shared__ __align__(16) float s_B[NP * kBcStride];
  __shared__ __align__(16) float s_C[SUMMARY ? 4 : NP * kBcStride];
  __shared__ __align__(16) float s_y[SUMMARY ? 4 : CH * kPartStride];

  const int lane = threadIdx.x;
  const int row = lane >> 4;
  const int ci = lane & 15;
  const int64_t gpb = (p.dim + CH - 1) / CH;
  const int64_t b = blockIdx.x / gpb;
  const int64_t d0 = (blockIdx.x % gpb) * CH;
  const int seg = blockIdx.y;
  const int64_t t_begin = (int64_t)seg * p.seg_len;
  const int64_t t_end = min(p.L, t_begin + p.seg_len);
  const bool fast_ok = p.vec_io != 0 && p.bc_vec != 0;
  const bool has_z = !SUMMARY && Z != nullptr;
  const bool softplus = p.softplus != 0;
  const int64_t grp = d0 / (p.dim / p.ngroups);
  const IO* __restrict__ Bg = Bm + b * p.B_sb + grp * p.B_sg;
  const IO* __restrict__ Cg = Cm + b * p.C_sb + grp * p.C_sg;
  const int n0 = row * NS;

  // ---- per-lane constants of channel d = d0 + ci, states n0 .. n0 + NS - 1
  const int64_t d = d0 + ci;
  const bool live = d < p.dim;
  float ap[HEAD ? 1 : NS];
  if constexpr (HEAD) {
    ap[0] = live ? Am[d / p.headdim] * kLog2e : 0.0f;
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      ap[j] = (live && n0 + j < p.N) ? Am[d * p.N + n0 + j] * kLog2e : 0.0f;
  }
  float h[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) h[j] = 0.0f;
  if (!SUMMARY && seg > 0 && live) {
    const int64_t base = (b * p.dim + d) * p.nseg;
    for (int s = 0; s < seg; ++s) {
      const float ds = dsum[base + s];
      const float* he = hend + (base + s) * p.N;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float a;
        if constexpr (HEAD) a = ap[0]; else a = ap[j];
        if (n0 + j < p.N) h[j] = __builtin_amdgcn_exp2f(a * ds) * h[j] + he[n0 + j];
      }
    }
  }
  double dsum_total = 0.0;

  // ---- this lane's prologue/epilogue items, fixed for the whole segment: io item it covers
  // channel row ir[it], steps itl[it] .. +V of each tile; B/C item it covers state bn[it]
  const IO* xrow[IPT];
  const IO* drow_p[IPT];
  const IO* zrow[IPT];
  IO* yrow[IPT];
  float ibias[IPT], iD[IPT];
  int ir[IPT], itl[IPT];
  bool ilive[IPT];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int item = lane + it * 64;
    ir[it] = item / CPR;
    itl[it] = (item % CPR) * V;
    const int64_t dd = d0 + ir[it];
    ilive[it] = dd < p.dim;
    const int64_t dv = min(dd, p.dim - 1);  // rows past dim read a valid row (never stored)
    const int64_t dr = HEAD ? dv / p.headdim : dv;
    xrow[it] = X + b * p.x_sb + dv * p.x_sd;
    drow_p[it] = DL + b * p.dl_sb + dr * p.dl_sd;
    zrow[it] = has_z ? Z + b * p.z_sb + dv * p.z_sd : nullptr;
    yrow[it] = SUMMARY ? nullptr : Y + b * p.y_sb + dv * p.y_sd;
    ibias[it] = bias_p ? bias_p[dr] : 0.0f;
    iD[it] = (!SUMMARY && Dm) ? Dm[dv] : 0.0f;
  }
  const IO* brow[BPT];
  const IO* crow[BPT];
  int bn[BPT], btl[BPT];
#pragma unroll
  for (int it = 0; it < BPT; ++it) {
    const int item = lane + it * 64;
    bn[it] = item / CPR;
    btl[it] = (item % CPR) * V;
    const int64_t nn = min<int64_t>(bn[it], p.N - 1);
    brow[it] = Bg + nn * p.B_sn;
    crow[it] = SUMMARY ? nullptr : Cg + nn * p.C_sn;
  }

  // raw 16-byte words of the next full tile
  u32x4 rx[IPT], rd[IPT], rz[IPT], rb[BPT], rc[BPT];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      rx[it] = load16<true>(xrow[it] + t0 + itl[it]);
      rd[it] = load16<true>(drow_p[it] + t0 + itl[it]);
      if (has_z) rz[it] = load16<true>(zrow[it] + t0 + itl[it]);
    }
#pragma unroll
    for (int it = 0; it < BPT; ++it) {
      rb[it] = load16<false>(brow[it] + t0 + btl[it]);
      if (!SUMMARY) rc[it] = load16<false>(crow[it] + t0 + btl[it]);
    }
  };
  if (fast_ok && t_end - t_begin >= kTB) fetch(t_begin);

  float xkeep[IPT][V];
  u32x4 zkeep[IPT];

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTB) {
    const int tb_len = (int)min<int64_t>(kTB, t_end - t0);
    const bool full = fast_ok && tb_len == kTB;

    // ---- prologue: delta, u = delta * x into LDS; B, C tiles into LDS (fp32)
    if (full) {
#pragma unroll
      for (int it = 0; it < IPT; ++it) {
        float dv[V];
        unpack16<IO>(rx[it], xkeep[it]);
        unpack16<IO>(rd[it], dv);
        zkeep[it] = rz[it];
        float du[2 * V];
        if (softplus) {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const float dl = softplus_f32(dv[e] + ibias[it]);
            du[2 * e] = dl;
            du[2 * e + 1] = dl * xkeep[it][e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const float dl = dv[e] + ibias[it];
            du[2 * e] = dl;
            du[2 * e + 1] = dl * xkeep[it][e];
          }
        }
        float4* dst = reinterpret_cast<float4*>(&s_du[ir[it] * kDuStride + 2 * itl[it]]);
#pragma unroll
        for (int k = 0; k < V / 2; ++k)
          dst[k] = make_float4(du[4 * k], du[4 * k + 1], du[4 * k + 2], du[4 * k + 3]);
      }
#pragma unroll
      for (int it = 0; it < BPT; ++it) {
        float bv[V], cv[V];
        unpack16<IO>(rb[it], bv);
        if constexpr (!SUMMARY) unpack16<IO>(rc[it], cv);
        if (bn[it] >= p.N) {
#pragma unroll
          for (int e = 0; e < V; ++e) { bv[e] = 0.0f; cv[e] = 0.0f; }
        }
        float4* db = reinterpret_cast<float4*>(&s_B[bn[it] * kBcStride + btl[it]]);
#pragma unroll
        for (int k = 0; k < V / 4; ++k)
          db[k] = make_float4(bv[4 * k], bv[4 * k + 1], bv[4 * k + 2], bv[4 * k + 3]);
        if constexpr (!SUMMARY) {
          float4* dc = reinterpret_cast<float4*>(&s_C[bn[it] * kBcStride + btl[it]]);
#pragma unroll
          for (int k = 0; k < V / 4; ++k)
            dc[k] = make_float4(cv[4 * k], cv[4 * k + 1], cv[4 * k + 2], cv[4 * k + 3]);
        }
      }
      // the raw registers are free: start loading the next tile
      if (t_end - (t0 + kTB) >= kTB) fetch(t0 + kTB);
    } else {
      // partial tile or unaligned rows: guarded element loads; padding steps and channels get
      // delta = u = 0 (dA = 1, dB x = 0) and B = C = 0
#pragma unroll
      for (int it = 0; it < IPT; ++it) {
        const int cnt = max(0, min(V, tb_len - itl[it]));
        const int c2 = ilive[it] ? cnt : 0;
        float dv[V], zv[V];
        load_chunk<IO, true>(xrow[it], t0 + itl[it], c2, false, xkeep[it]);
        load_chunk<IO, true>(drow_p[it], t0 + itl[it], c2, false, dv);
        if (has_z) load_chunk<IO, true>(zrow[it], t0 + itl[it], c2, false, zv);
        else {
#pragma unroll
          for (int e = 0; e < V; ++e) zv[e] = 0.0f;
        }
        uint32_t zw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (V == 8) zw[k] = pack_bf16x2(zv[2 * k], zv[2 * k + 1]);
          else zw[k] = __float_as_uint(zv[k]);
        }
        zkeep[it] = u32x4{zw[0], zw[1], zw[2], zw[3]};
        float du[2 * V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float v = dv[e] + ibias[it];
          float dl = softplus ? softplus_f32(v) : v;
          if (e >= c2) dl = 0.0f;
          du[2 * e] = dl;
          du[2 * e + 1] = dl * xkeep[it][e];
        }
        float4* dst = reinterpret_cast<float4*>(&s_du[ir[it] * kDuStride + 2 * itl[it]]);
#pragma unroll
        for (int k = 0; k < V / 2; ++k)
          dst[k] = make_float4(du[4 * k], du[4 * k + 1], du[4 * k + 2], du[4 * k + 3]);
      }
#pragma unroll
      for (int it = 0; it < BPT; ++it) {
        const int cnt = bn[it] < p.N ? max(0, min(V, tb_len - btl[it])) : 0;
        float bv[V], cv[V];
        load_chunk<IO, false>(brow[it], t0 + btl[it], cnt, false, bv);
        if constexpr (!SUMMARY) load_chunk<IO, false>(crow[it], t0 + btl[it], cnt, false, cv);
        float4* db = reinterpret_cast<float4*>(&s_B[bn[it] * kBcStride + btl[it]]);
#pragma unroll
        for (int k = 0; k < V / 4; ++k)
          db[k] = make_float4(bv[4 * k], bv[4 * k + 1], bv[4 * k + 2], bv[4 * k + 3]);
        if constexpr (!SUMMARY) {
          float4* dc = reinterpret_cast<float4*>(&s_C[bn[it] * kBcStride + btl[it]]);
#pragma unroll
          for (int k = 0; k < V / 4; ++k)
            dc[k] = make_float4(cv[4 * k], cv[4 * k + 1], cv[4 * k + 2], cv[4 * k + 3]);
        }
      }
      if (fast_ok && t0 + kTB < t_end && t_end - (t0 + kTB) >= kTB) fetch(t0 + kTB);
    }
    __syncthreads();

    // ---- recurrence over the tile
    for (int tt = 0; tt < tb_len; tt += 8) {
      float dl[8], u[8];
      const float4* src = reinterpret_cast<const float4*>(&s_du[ci * kDuStride + 2 * tt]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = src[k];
        dl[2 * k] = q.x; u[2 * k] = q.y; dl[2 * k + 1] = q.z; u[2 * k + 1] = q.w;
      }
      float acc[8];
      float dA_head[HEAD ? 8 : 1];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[k] = 0.0f;
        if constexpr (HEAD) dA_head[k] = __builtin_amdgcn_exp2f(dl[k] * ap[0]);
      }
      if constexpr (SUMMARY) {
        float s8 = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s8 += dl[k];
        dsum_total += (double)s8;
      }
#pragma unroll
      for (int jc = 0; jc < NS; jc += 4) {
        // 16 (state, step) values per register and row: states n0+jc .. +3, steps tt .. tt+3
        // (lo) and tt+4 .. tt+7 (hi)
        const int bc_off = (n0 + jc + (ci >> 2)) * kBcStride + tt + (ci & 3);
        const float b_lo = s_B[bc_off], b_hi = s_B[bc_off + 4];
        float c_lo = 0.0f, c_hi = 0.0f;
        if constexpr (!SUMMARY) { c_lo = s_C[bc_off]; c_hi = s_C[bc_off + 4]; }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int slot = j * 4 + (k & 3);
            float dA;
            if constexpr (HEAD) dA = dA_head[k]; else dA = __builtin_amdgcn_exp2f(dl[k] * ap[jc + j]);
            const float bb = row_bcast_k(k < 4 ? b_lo : b_hi, slot);
            h[jc + j] = fmaf(dA, h[jc + j], u[k] * bb);
            if constexpr (!SUMMARY) {
              const float cc2 = row_bcast_k(k < 4 ? c_lo : c_hi, slot);
              acc[k] = fmaf(cc2, h[jc + j], acc[k]);
            }
          }
        }
      }
      if constexpr (!SUMMARY) {
        const float y_lo = rows_transpose_sum4(acc[0], acc[1], acc[2], acc[3]);
        const float y_hi = rows_transpose_sum4(acc[4], acc[5], acc[6], acc[7]);
        s_y[ci * kPartStride + tt + row] = y_lo;
        s_y[ci * kPartStride + tt + 4 + row] = y_hi;
      }
    }
    __syncthreads();

    // ---- epilogue: y = (readout + D x) * silu(z), 16-byte stores
    if constexpr (!SUMMARY) {
#pragma unroll
      for (int it = 0; it < IPT; ++it) {
        float yv[V];
#pragma unroll
        for (int e4 = 0; e4 < V; e4 += 4) {
          const float4 s4 = *reinterpret_cast<const float4*>(&s_y[ir[it] * kPartStride + itl[it] + e4]);
          yv[e4] = s4.x; yv[e4 + 1] = s4.y; yv[e4 + 2] = s4.z; yv[e4 + 3] = s4.w;
        }
        float zv[V];
        unpack16<IO>(zkeep[it], zv);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          float yy = fmaf(iD[it], xkeep[it][e], yv[e]);
          if (has_z) yy *= silu_f32(zv[e]);
          yv[e] = yy;
        }
        if (full) {
          if (ilive[it]) store_chunk<IO>(yrow[it], t0 + itl[it], V, true, yv);
        } else {
          const int cnt = max(0, min(V, tb_len - itl[it]));
          if (ilive[it] && cnt > 0) store_chunk<IO>(yrow[it], t0 + itl[it], cnt, false, yv);
        }
      }
    }
  }

  if constexpr (SUMMARY) {
    if (live) {
      const int64_t base = (b * p.dim + d) * p.nseg + seg;
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (n0 + j < p.N) hend[base * p.N + n0 + j] = h[j];
      if (row == 0) dsum[base] = (float)dsum_total;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// host-side launch

#define SCAN_ARGS(p)                                                                         \
  static_cast<const IO*>(p.x), static_cast<const IO*>(p.delta), static_cast<const IO*>(p.B), \
      static_cast<const IO*>(p.C), static_cast<const IO*>(p.z), static_cast<IO*>(p.y), p.A,  \
      p.D, p.delta_bias, p.hend, p.dsum, p

template <typename IO, int NS, int NW, bool HEAD>
static hipError_t launch_cfg(const ScanParams& p, hipStream_t stream) {
  const dim3 block(64 * NW);
  const int64_t groups = p.batch * p.groups_per_batch;
  if (p.nseg > 1) {
    const dim3 grid_sum((unsigned)groups, (unsigned)(p.nseg - 1));
    hipLaunchKernelGGL((scan_fwd_kernel<IO, NS, NW, HEAD, true>), grid_sum, block, 0, stream,
                       SCAN_ARGS(p));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)groups, (unsigned)p.nseg);
  hipLaunchKernelGGL((scan_fwd_kernel<IO, NS, NW, HEAD, false>), grid, block, 0, stream,
                     SCAN_ARGS(p));
  return hipGetLastError();
}

template <typename IO, int NS, bool HEAD>
static hipError_t launch_rows(const ScanParams& p, hipStream_t stream) {
  const dim3 block(64);
  const int64_t groups = p.batch * ((p.dim + 15) / 16);
  if (p.nseg > 1) {
    const dim3 grid_sum((unsigned)groups, (unsigned)(p.nseg - 1));
    hipLaunchKernelGGL((scan_rows_kernel<IO, NS, HEAD, true>), grid_sum, block, 0, stream,
                       SCAN_ARGS(p));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)groups, (unsigned)p.nseg);
  hipLaunchKernelGGL((scan_rows_kernel<IO, NS, HEAD, false>), grid, block, 0, stream,
                     SCAN_ARGS(p));
  return hipGetLastError();
}

template <typename IO, bool HEAD>
static hipError_t launch_n(const ScanParams& p, hipStream_t stream) {
  const int64_t N = p.N;
  if (N <= 16) return launch_rows<IO, 4, HEAD>(p, stream);
  if (N <= 32) return launch_rows<IO, 8, HEAD>(p, stream);
  if (N <= 64) return launch_cfg<IO, 16, 4, HEAD>(p, stream);
  return launch_cfg<IO, 16, 8, HEAD>(p, stream);  // N <= 128 (checked by the caller)
}

hipError_t launch_scan_fwd(const ScanParams& p, bool bf16, bool head, hipStream_t stream) {
  if (bf16) return head ? launch_n<bf16_bits, true>(p, stream) : launch_n<bf16_bits, false>(p, stream);
  return head ? launch_n<float, true>(p, stream) : launch_n<float, false>(p, stream);
}

int time_tile() { return kTB; }

// Channels per workgroup of the kernel that launch_scan_fwd picks for dstate N.
int channels_per_group(int64_t N) { return N <= 32 ? 16 : kChannelsPerGroup; }

}  // namespace ssm
