// Chunked matrix form of the scalar-decay selective scan on the gfx950 matrix cores.
//
// "Transformers are SSMs" review page, proposed method: the scan is multiplication by a
// semiseparable matrix, and a block decomposition of that matrix trades the recurrence for dense
// products. With one decay per head, a_t = delta_t * A, and a chunk of kQ steps that starts from
// the state H (N states x P channels), let s_t = a_0 + ... + a_t (inclusive, within the chunk)
// and w_t the input weight (delta_t, or the zero-order-hold weight). Then
//   Y[t][p] = e^{s_t} sum_n C[n][t] H[n][p]                                (off-diagonal blocks)
//           + sum_{j<=t} (sum_n C[n][t] B[n][j]) e^{s_t - s_j} w_j x[p][j]  (diagonal block)
//   H'[n][p] = e^{s_Q} H[n][p] + sum_j B[n][j] e^{s_Q - s_j} w_j x[p][j]    (state passed on)
// which is the recurrence h_t = e^{a_t} h_{t-1} + w_t B_t x_t, y_t = C_t . h_t unrolled over the
// chunk. Every sum over n or j is a product of 64 x 64 x {64, 128} tiles, computed by the
// 16x16x32 bf16 MFMA with fp32 accumulation; H stays in fp32 accumulators for the whole sequence.
// B, C and x enter as the exact bf16 inputs. The operands computed in fp32 (the decay-weighted
// C.B tile, the state H, the weighted inputs) enter as two bf16 terms hi + lo, hi = bf16(v) and
// lo = bf16(v - hi), which carry 16 significant bits: one bf16 rounding of these operands makes
// errors of the order of 1e-2 relative to the output in the max norm, the pair brings the error
// down to that of rounding y itself to bf16.
//
// Work decomposition: one workgroup = one batch entry x 64 channels of one head (P = 64), four
// wavefronts, the whole sequence in order. Wavefront w owns channels p in [16w, 16w + 16) and all
// N states of H for them (N/16 accumulator tiles). Per chunk:
//   1. G^T[j][t] = sum_n B[n][j] C[n][t] for the 10 causal 16x16 tiles (split over the
//      wavefronts), masked, scaled by e^{s_t - s_j} w_j and stored as bf16 hi and lo parts in
//      LDS (Lmat[t][j]).
//   2. Y = (e^{s_t} (C^T H)) + Lmat x for the wavefront's channels; H enters as the B operand
//      straight from its accumulators (the k-slot order of the operand is chosen to match the
//      accumulator layout, and C^T is read in the same order).
//   3. y = (Y + D x) silu(z), stored as bf16.
//   4. H = e^{s_Q} H + B (e^{s_Q - s_j} w_j x).
// The B and C tiles of a chunk are staged in LDS (transposed for the products over n, plain for
// the product over j) while the next chunk's global loads are in flight; LDS is double buffered.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16, c = l % 16): A operand holds
// A[c][8g .. 8g+8), B operand holds B[8g .. 8g+8)[c], the accumulator holds D[4g .. 4g+4)[c].
// Output rows of the Y tiles are permuted so that lane (g, c) ends up with the 16 consecutive
// steps [16g, 16g+16) of channel 16w + c: x, z and y then move 32 contiguous bytes per lane.
#include "scan_kernels.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 64;   // steps per chunk
constexpr int kPB = 64;  // channels per workgroup
constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mma(const u32x4 a, const u32x4 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// (a, b) -> {hi, lo}: packed bf16 pairs hi = bf16(a, b) and lo = bf16 of the remainders (the
// remainders are exact in fp32)
__device__ __forceinline__ u32x2 split2(float a, float b) {
  const uint32_t hi = pack_bf16x2(a, b);
  return u32x2{hi, pack_bf16x2(a - lo_f(hi), b - hi_f(hi))};
}

// LDS byte offsets. Each swizzle permutes the 16-byte slots within a row so that the eight
// lanes of one ds_read_b128 / ds_write_b128 phase hit distinct bank groups.
//   transposed B / C tiles [t][n] (row = 2N bytes): slot ^ ((t ^ t >> 3) & 7)
//   plain B tile [n][j] (row = 128 bytes):          slot ^ ((n ^ n >> 3) & 7)
//   Lmat [t][j] (row = 128 bytes):                  slot ^ ((t ^ (t >> 2 & 4)) & 7)
template <int N>
__device__ __forceinline__ int off_tr(int t, int slot) {
  return t * (2 * N) + ((slot ^ ((t ^ (t >> 3)) & 7)) << 4);
}
__device__ __forceinline__ int off_bn(int n, int slot) {
  return n * 128 + ((slot ^ ((n ^ (n >> 3)) & 7)) << 4);
}
__device__ __forceinline__ int off_lm(int t, int slot) {
  return t * 128 + ((slot ^ ((t ^ ((t >> 2) & 4)) & 7)) << 4);
}

__device__ __forceinline__ u32x4 lds16(const uint8_t* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ u32x2 lds8(const uint8_t* base, int off) {
  return *reinterpret_cast<const u32x2*>(base + off);
}
__device__ __forceinline__ void sts16(uint8_t* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

// The 16-byte word of a row at [t, t + 8), t a multiple of 8 and the row 16-byte aligned, with
// one aligned 16-byte load whatever t: a word that reaches past L is still read whole (an
// aligned 16-byte block that holds a valid element lies in that element's page), and a word
// wholly past L is replaced by the word that holds element L - 1. Every chunk thus issues the
// same loads into the same registers, ragged last chunk or not; mask8 zeroes the elements at or
// past L when the word is used (not here, which would make the load wait for its data).
template <bool STREAM>
__device__ __forceinline__ u32x4 load8(const bf16_bits* row, int64_t t, int64_t L) {
  return load16<STREAM>(row + (t < L ? t : ((L - 1) & ~(int64_t)7)));
}
// w with the elements at index >= nv zeroed (nv = valid elements of the word; <= 0: none)
__device__ __forceinline__ u32x4 mask8(const u32x4 w, int64_t nv) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t keep = nv >= 2 * k + 2 ? 0xffffffffu : (nv == 2 * k + 1 ? 0x0000ffffu : 0u);
    r[k] = w[k] & keep;
  }
  return r;
}

// Per-chunk step arrays in LDS, kQ floats each: s2 = s_t log2 e, w = w_t, es = e^{s_t},
// cw = e^{s_Q - s_t} w_t.
struct StepArrays {
  float s2[kQ];
  float w[kQ];
  float es[kQ];
  float cw[kQ];
};

// GATE: y is multiplied by silu(z).
template <int N, bool GATE>
__global__ void __launch_bounds__(kThreads, 1)
    ssd_fwd_kernel(const bf16_bits* __restrict__ X, const bf16_bits* __restrict__ DL,
                   const bf16_bits* __restrict__ Bm, const bf16_bits* __restrict__ Cm,
                   const bf16_bits* __restrict__ Z, bf16_bits* __restrict__ Yo,
                   const float* __restrict__ Am, const float* __restrict__ Dm,
                   const float* __restrict__ bias_p, const ScanParams p) {
  constexpr int NM = N / 16;           // state tiles of H per wavefront
  constexpr int NK = N / 32;           // k-steps of the products over n
  constexpr int NB = N / 8;            // 8-state blocks of a staged tile
  constexpr int kMat = kQ * 2 * N;     // bytes of one staged bf16 tile (N x kQ)
  constexpr int kBuf = 3 * kMat;       // transposed B, transposed C, plain B
  constexpr int kLm = kQ * kQ * 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kBuf + 2 * kLm];
  __shared__ StepArrays sa[2];
  uint8_t* const lm = smem + 2 * kBuf;   // Lmat hi parts
  uint8_t* const lml = lm + kLm;         // Lmat lo parts

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;

  // work item -> (batch entry, channel block). Workgroups are dispatched to the eight
  // accelerator dies round robin; consecutive items share B and C, so each die gets a
  // contiguous range of items and keeps one batch entry's B/C in its L2.
  const int64_t nblk = p.dim / kPB;
  const int64_t nwork = p.batch * nblk;
  int64_t item = blockIdx.x;
  if (nwork % 8 == 0) item = (item & 7) * (nwork >> 3) + (item >> 3);
  const int64_t b = item / nblk;
  const int64_t d0 = (item % nblk) * kPB;
  const int64_t head = d0 / p.headdim;
  const int64_t grp = d0 / (p.dim / p.ngroups);
  const int64_t L = p.L;
  const int64_t nchunks = (L + kQ - 1) / kQ;

  const float a_log2 = Am[head] * kLog2e;
  const float bias = bias_p ? bias_p[head] : 0.0f;
  const bool softplus = p.softplus != 0;
  const bool zoh = p.zoh != 0;

  // this lane's channel and rows
  const int pl = 16 * wave + c;
  const int64_t d = d0 + pl;
  const bf16_bits* xrow = X + b * p.x_sb + d * p.x_sd;
  const bf16_bits* zrow = GATE ? Z + b * p.z_sb + d * p.z_sd : nullptr;
  bf16_bits* yrow = Yo + b * p.y_sb + d * p.y_sd;
  const bf16_bits* dlrow = DL + b * p.dl_sb + head * p.dl_sd;
  const float Dp = Dm ? Dm[d] : 0.0f;

  // staging role: thread -> one 8 x 8 block (8 states x 8 steps) of B (mat 0) or C (mat 1).
  // With N = 64 there are 128 blocks for 256 threads: the upper half of the threads loads the
  // blocks of the lower half again (L2 hits) and writes nothing, so every load is unconditional.
  constexpr int kBlocks = 2 * N;
  const int blk = tid % kBlocks;
  const bool stager = kBlocks == kThreads || tid < kBlocks;  // uniform per wavefront
  const int mat = blk / (8 * NB);
  const int nb = blk % NB;
  const int tb = (blk % (8 * NB)) / NB;
  const bf16_bits* bcrow = (mat == 0 ? Bm + b * p.B_sb + grp * p.B_sg + (int64_t)(8 * nb) * p.B_sn
                                     : Cm + b * p.C_sb + grp * p.C_sg + (int64_t)(8 * nb) * p.C_sn);
  const int64_t bc_sn = mat == 0 ? p.B_sn : p.C_sn;

  // state accumulators: H[m][q] = H[n = 16m + 4g + q][p = 16 wave + c]
  f32x4 H[NM];
  if (p.h0) {
    const float* hp = p.h0 + (b * p.dim + d) * N + 4 * g;
#pragma unroll
    for (int m = 0; m < NM; ++m) H[m] = *reinterpret_cast<const f32x4*>(hp + 16 * m);
  } else {
#pragma unroll
    for (int m = 0; m < NM; ++m) H[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // the strictly upper 16x16 tiles of Lmat are never written: zero them once
  for (int i = tid; i < kQ * kQ / 8; i += kThreads) {
    const int t = i / (kQ / 8), slot = i % (kQ / 8);
    if (2 * (t / 16) + 1 < slot) {
      sts16(lm, off_lm(t, slot), u32x4{0, 0, 0, 0});
      sts16(lml, off_lm(t, slot), u32x4{0, 0, 0, 0});
    }
  }

  // Loads of a chunk into registers (load8: the same instructions for every chunk). B/C go to
  // pbc and delta to pdl, which stage() moves into LDS one chunk later; x and z go to one of two
  // register sets that the chunks use alternately, so a set is read one chunk after its loads
  // were issued and never copied.
  u32x4 pbc[8];
  bf16_bits pdl = 0;
  auto issue_bc = [&](int64_t ch) __attribute__((always_inline)) {
    const int64_t t0 = ch * kQ;
#pragma unroll
    for (int r = 0; r < 8; ++r) pbc[r] = load8<false>(bcrow + r * bc_sn, t0 + 8 * tb, L);
    const int64_t t = t0 + lane;
    pdl = dlrow[t < L ? t : L - 1];  // past L: masked when staged
  };
  auto issue_xz = [&](int64_t ch, u32x4 (&xr)[2], u32x4 (&zr)[2]) __attribute__((always_inline)) {
    const int64_t t = ch * kQ + 16 * g;
#pragma unroll
    for (int s = 0; s < 2; ++s) xr[s] = load8<true>(xrow, t + 8 * s, L);
    if constexpr (GATE) {
#pragma unroll
      for (int s = 0; s < 2; ++s) zr[s] = load8<true>(zrow, t + 8 * s, L);
    }
  };
  // pbc / pdl -> LDS buffer `buf`: transposed and plain tiles, and the step arrays
  auto stage = [&](int buf, int64_t ch) __attribute__((always_inline)) {
    uint8_t* base = smem + buf * kBuf;
    const int64_t nv = L - (ch * kQ + 8 * tb);
#pragma unroll
    for (int r = 0; r < 8; ++r) pbc[r] = mask8(pbc[r], nv);
    if (stager) {
      uint8_t* tr = base + mat * kMat;
      // transpose the 8x8 block: output row (step) e holds states 8nb .. 8nb+8
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t r0 = pbc[2 * k][e >> 1], r1 = pbc[2 * k + 1][e >> 1];
          w[k] = (e & 1) ? ((r0 >> 16) | (r1 & 0xffff0000u)) : ((r0 & 0xffffu) | (r1 << 16));
        }
        sts16(tr, off_tr<N>(8 * tb + e, nb), u32x4{w[0], w[1], w[2], w[3]});
      }
      if (mat == 0) {
        uint8_t* bn = base + 2 * kMat;
#pragma unroll
        for (int r = 0; r < 8; ++r) sts16(bn, off_bn(8 * nb + r, tb), pbc[r]);
      }
    }
    if (wave == 3) {
      const int64_t t = ch * kQ + lane;
      const bool valid = t < L;
      float dl = to_f32(pdl) + bias;
      if (softplus) dl = softplus_f32(dl);
      float a2 = dl * a_log2;  // a_t log2 e
      float w = dl;
      if (zoh) w = dl * zoh_ratio(__builtin_amdgcn_exp2f(a2), a2);
      if (!valid) { a2 = 0.0f; w = 0.0f; }
      // inclusive prefix sum over the 64 steps of the chunk
      float s2 = a2;
#pragma unroll
      for (int k = 1; k < 64; k <<= 1) {
        const float o = __shfl_up(s2, k, 64);
        if (lane >= k) s2 += o;
      }
      const float sQ = __shfl(s2, 63, 64);
      StepArrays& A = sa[buf];
      A.s2[lane] = s2;
      A.w[lane] = w;
      A.es[lane] = __builtin_amdgcn_exp2f(s2);
      A.cw[lane] = __builtin_amdgcn_exp2f(sQ - s2) * w;
    }
  };

  // G^T tile k of the 10 causal tiles (jt <= tt), in the order (0,0) (0,1) (0,2) (0,3) (1,1)
  // (1,2) (1,3) (2,2) (2,3) (3,3): masked, decay-weighted, split and stored into Lmat.
  auto tile_jt = [](int k) { return k < 4 ? 0 : (k < 7 ? 1 : (k < 9 ? 2 : 3)); };
  auto tile_tt = [](int k, int jt) { return jt + k - (jt == 0 ? 0 : (jt == 1 ? 4 : (jt == 2 ? 7 : 9))); };
  auto store_lmat = [&](const StepArrays& A, int jt, int tt, const f32x4 acc)
      __attribute__((always_inline)) {
    // acc[q] = G^T[j = 16jt + 4g + q][t = 16tt + c]
    const int t = 16 * tt + c;
    const int j0 = 16 * jt + 4 * g;
    const float st = A.s2[t];
    const f32x4 sj = *reinterpret_cast<const f32x4*>(&A.s2[j0]);
    const f32x4 wj = *reinterpret_cast<const f32x4*>(&A.w[j0]);
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = (j0 + q <= t) ? acc[q] * __builtin_amdgcn_exp2f(st - sj[q]) * wj[q] : 0.0f;
    const u32x2 s01 = split2(v[0], v[1]), s23 = split2(v[2], v[3]);
    const int o = off_lm(t, 2 * jt + (g >> 1)) + 8 * (g & 1);
    *reinterpret_cast<u32x2*>(lm + o) = u32x2{s01[0], s23[0]};
    *reinterpret_cast<u32x2*>(lml + o) = u32x2{s01[1], s23[1]};
  };

  auto chunk = [&](int64_t ch, const int buf, u32x4 (&xr)[2], u32x4 (&zr)[2])
      __attribute__((always_inline)) {
    u32x4 xv[2], zv[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      xv[s] = mask8(xr[s], L - (ch * kQ + 16 * g + 8 * s));
      if constexpr (GATE) zv[s] = mask8(zr[s], L - (ch * kQ + 16 * g + 8 * s));
    }
    const uint8_t* base = smem + buf * kBuf;
    const uint8_t* bt = base;
    const uint8_t* ct = base + kMat;
    const uint8_t* bn = base + 2 * kMat;
    const StepArrays& A = sa[buf];
    const int64_t t0 = ch * kQ;

    // 1. Lmat: tiles wave and wave + 4 for every wavefront, wave + 8 for wavefronts 0 and 1
    {
      const int jt0 = tile_jt(wave), tt0 = tile_tt(wave, jt0);
      const int jt1 = tile_jt(wave + 4), tt1 = tile_tt(wave + 4, jt1);
      u32x4 a0[NK], b0[NK], a1[NK], b1[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        a0[kk] = lds16(bt, off_tr<N>(16 * jt0 + c, 4 * kk + g));
        b0[kk] = lds16(ct, off_tr<N>(16 * tt0 + c, 4 * kk + g));
        a1[kk] = lds16(bt, off_tr<N>(16 * jt1 + c, 4 * kk + g));
        b1[kk] = lds16(ct, off_tr<N>(16 * tt1 + c, 4 * kk + g));
      }
      f32x4 g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        g0 = mma(a0[kk], b0[kk], g0);
        g1 = mma(a1[kk], b1[kk], g1);
      }
      store_lmat(A, jt0, tt0, g0);
      store_lmat(A, jt1, tt1, g1);
      if (wave < 2) {
        const int jt2 = tile_jt(wave + 8), tt2 = tile_tt(wave + 8, jt2);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          a0[kk] = lds16(bt, off_tr<N>(16 * jt2 + c, 4 * kk + g));
          b0[kk] = lds16(ct, off_tr<N>(16 * tt2 + c, 4 * kk + g));
        }
        f32x4 g2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) g2 = mma(a0[kk], b0[kk], g2);
        store_lmat(A, jt2, tt2, g2);
      }
    }
    __syncthreads();

    // 2. Y tiles i = 0..3: row r of tile i is step 16 (r / 4) + 4i + r % 4. First the
    //    inter-chunk part e^{s_t} C^T H, then the intra-chunk part Lmat x.
    f32x4 Y[4];
    {
      int tr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tr[i] = 16 * (c >> 2) + 4 * i + (c & 3);
        Y[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        // k-slots: states 32kk + 4g + (0..3), then 32kk + 16 + 4g + (0..3)
        const u32x2 h01 = split2(H[2 * kk][0], H[2 * kk][1]), h23 = split2(H[2 * kk][2], H[2 * kk][3]);
        const u32x2 h45 = split2(H[2 * kk + 1][0], H[2 * kk + 1][1]);
        const u32x2 h67 = split2(H[2 * kk + 1][2], H[2 * kk + 1][3]);
        const u32x4 hb = {h01[0], h23[0], h45[0], h67[0]};
        const u32x4 hl = {h01[1], h23[1], h45[1], h67[1]};
        u32x4 ca[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 4 * kk + (g >> 1);
          const u32x2 lo = lds8(ct, off_tr<N>(tr[i], slot) + 8 * (g & 1));
          const u32x2 hi = lds8(ct, off_tr<N>(tr[i], slot + 2) + 8 * (g & 1));
          ca[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = mma(ca[i], hb, Y[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = mma(ca[i], hl, Y[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[i] *= *reinterpret_cast<const f32x4*>(&A.es[16 * g + 4 * i]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 la[4], ll[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          la[i] = lds16(lm, off_lm(tr[i], 2 * g + s));
          ll[i] = lds16(lml, off_lm(tr[i], 2 * g + s));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = mma(la[i], xv[s], Y[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = mma(ll[i], xv[s], Y[i]);
      }
    }

    // 3. epilogue: lane holds steps 16g + 4i + q of channel pl
    {
      uint32_t out[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * i + q;  // step within the lane's 16
          const uint32_t xw = xv[e >> 3][(e & 7) >> 1];
          const float xe = (e & 1) ? hi_f(xw) : lo_f(xw);
          float yy = Y[i][q] + Dp * xe;
          if constexpr (GATE) {
            const uint32_t zw = zv[e >> 3][(e & 7) >> 1];
            yy *= silu_f32((e & 1) ? hi_f(zw) : lo_f(zw));
          }
          v[q] = yy;
        }
        out[2 * i] = pack_bf16x2(v[0], v[1]);
        out[2 * i + 1] = pack_bf16x2(v[2], v[3]);
      }
      const int64_t ts = t0 + 16 * g;
      if (t0 + kQ <= L) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x4 o = {out[4 * s], out[4 * s + 1], out[4 * s + 2], out[4 * s + 3]};
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(yrow + ts + 8 * s));
        }
      } else {
        for (int e = 0; e < 16; ++e)
          if (ts + e < L) yrow[ts + e] = (bf16_bits)((out[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      }
    }

    // 4. state update: H = e^{s_Q} H + B (cw x)
    {
      u32x4 xs[2], xl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(&A.cw[16 * g + 8 * s]);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(&A.cw[16 * g + 8 * s + 4]);
        const float cw[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        u32x2 sp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          sp[k] = split2(lo_f(xv[s][k]) * cw[2 * k], hi_f(xv[s][k]) * cw[2 * k + 1]);
        xs[s] = u32x4{sp[0][0], sp[1][0], sp[2][0], sp[3][0]};
        xl[s] = u32x4{sp[0][1], sp[1][1], sp[2][1], sp[3][1]};
      }
      const float eQ = A.es[kQ - 1];
#pragma unroll
      for (int m = 0; m < NM; ++m) H[m] *= eQ;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 ba[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) ba[m] = lds16(bn, off_bn(16 * m + c, 2 * g + s));
#pragma unroll
        for (int m = 0; m < NM; ++m) H[m] = mma(ba[m], xs[s], H[m]);
#pragma unroll
        for (int m = 0; m < NM; ++m) H[m] = mma(ba[m], xl[s], H[m]);
      }
    }

    // 5. the next chunk's B/C into the other buffer, then this register set's next loads
    if (ch + 1 < nchunks) stage(buf ^ 1, ch + 1);
    if (ch + 2 < nchunks) {
      issue_bc(ch + 2);
      issue_xz(ch + 2, xr, zr);
    }
    __syncthreads();
  };

  u32x4 xa[2], za[2], xb[2], zb[2];
  issue_bc(0);
  issue_xz(0, xa, za);
  stage(0, 0);
  if (nchunks > 1) {
    issue_bc(1);
    issue_xz(1, xb, zb);
  }
  __syncthreads();
  for (int64_t ch = 0; ch < nchunks; ch += 2) {
    chunk(ch, 0, xa, za);
    if (ch + 1 >= nchunks) break;
    chunk(ch + 1, 1, xb, zb);
  }

  if (p.hfin) {
    float* hp = p.hfin + (b * p.dim + d) * N + 4 * g;
#pragma unroll
    for (int m = 0; m < NM; ++m) *reinterpret_cast<f32x4*>(hp + 16 * m) = H[m];
  }
}

template <int N>
hipError_t launch_ssd_n(const ScanParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.batch * (p.dim / kPB))), block(kThreads);
  const bf16_bits* X = static_cast<const bf16_bits*>(p.x);
  const bf16_bits* DL = static_cast<const bf16_bits*>(p.delta);
  const bf16_bits* Bm = static_cast<const bf16_bits*>(p.B);
  const bf16_bits* Cm = static_cast<const bf16_bits*>(p.C);
  const bf16_bits* Z = static_cast<const bf16_bits*>(p.z);
  bf16_bits* Y = static_cast<bf16_bits*>(p.y);
  if (p.z)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, true>), grid, block, 0, stream, X, DL, Bm, Cm, Z, Y,
                       p.A, p.D, p.delta_bias, p);
  else
    hipLaunchKernelGGL((ssd_fwd_kernel<N, false>), grid, block, 0, stream, X, DL, Bm, Cm, Z, Y,
                       p.A, p.D, p.delta_bias, p);
  return hipGetLastError();
}

}  // namespace

bool ssd_supported(const ScanParams& p) {
  return (p.N == 64 || p.N == 128) && p.headdim % kPB == 0 && p.dim % kPB == 0 &&
         (p.dim / p.ngroups) % kPB == 0 && p.vec_io && p.bc_vec &&
         p.batch * (p.dim / kPB) <= 0x7fffffff;
}

hipError_t launch_ssd(const ScanParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.L == 0) return hipSuccess;
  return p.N == 64 ? launch_ssd_n<64>(p, stream) : launch_ssd_n<128>(p, stream);
}

}  // namespace ssm
