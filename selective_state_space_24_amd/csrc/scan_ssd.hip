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
//   1. G^T[j][t] = sum_n B[n][j] C[n][t] for the 10 causal 16x16 tiles, masked, scaled by
//      e^{s_t - s_j} w_j and stored as bf16 hi and lo parts in LDS (Lmat[t][j]). The tiles are
//      split over the wavefronts so that a wavefront's tiles share one operand, which it reads
//      from LDS once: (0,0) (0,1) (0,2); (0,3) (1,3) (2,3); (1,1) (1,2); (2,2) (3,3).
//   2. Y = (e^{s_t} (C^T H)) + Lmat x for the wavefront's channels; H enters as the B operand
//      straight from its accumulators (the k-slot order of the operand is chosen to match the
//      accumulator layout, and C^T is read in the same order).
//   3. y = (Y + D x) silu(z), stored as bf16.
//   4. H = e^{s_Q} H + B (e^{s_Q - s_j} w_j x).
//
// Data movement: every input of a chunk (the B and C tiles, N rows of 64 steps; the x and z
// tiles, 64 channel rows of 64 steps; the 64 steps of delta) goes from global memory straight
// into LDS (16-byte direct loads, no registers), one chunk ahead, into one of two stage buffers.
// The products over n need B and C transposed (step-major); those operands are read with the LDS
// transpose read ds_read_b64_tr_b16: in each group of 16 lanes, lane i's slot q receives element
// i % 4 of the 8 bytes that lane 4q + i / 4 addressed. A lane that addresses 4 consecutive steps
// of state row n_q thus hands step (its first step + e) of row n_q to the lanes that own that
// step. The only wait for global memory is at the end of a chunk.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16, c = l % 16): A operand holds
// A[c][8g .. 8g+8), B operand holds B[8g .. 8g+8)[c], the accumulator holds D[4g .. 4g+4)[c].
// Output rows of the Y tiles are permuted so that lane (g, c) ends up with the 16 consecutive
// steps [16g, 16g+16) of channel 16w + c: x, z and y then move 32 contiguous bytes per lane.
#include <type_traits>

#include "scan_kernels.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

// LDS layouts (byte offsets). A staged tile is [n][64 steps] bf16, 128 bytes (8 slots of 16
// bytes) per state row; slot s of row n is stored at slot s ^ sw(n), sw(n) = 2 (n & 3) +
// (bit 0 ^ bit 2 of n). sw is one-to-one on n & 7, so the plain 16-byte reads of 8 consecutive
// rows hit distinct bank groups; the transpose reads of the C.B tile (4 rows x 32 bytes) get
// four distinct slot pairs; those of the inter-chunk product (4 rows x 4 slots, one half of
// each) get 8 distinct slots, i.e. no more than two lanes per bank.
__device__ __forceinline__ int sw_row(int n) { return ((n & 3) << 1) | ((n ^ (n >> 2)) & 1); }
__device__ __forceinline__ int off_st(int n, int slot) { return n * 128 + ((slot ^ sw_row(n)) << 4); }
// Lmat [t][j] (row = 128 bytes): slot ^ ((t ^ (t >> 2 & 4)) & 7)
__device__ __forceinline__ int off_lm(int t, int slot) {
  return t * 128 + ((slot ^ ((t ^ ((t >> 2) & 4)) & 7)) << 4);
}

__device__ __forceinline__ u32x4 lds16(const lds_u8* base, int off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + off);
}
__device__ __forceinline__ void sts16(lds_u8* base, int off, u32x4 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(base + off) = v;
}
__device__ __forceinline__ void sts8(lds_u8* base, int off, u32x2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(base + off) = v;
}
// transpose read of 4 bf16 (see the header comment for the lane mapping)
__device__ __forceinline__ u32x2 ldtr(const lds_u8* base, int off) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_s16x4*>(const_cast<lds_u8*>(base) + off));
  return __builtin_bit_cast(u32x2, v);
}

// The element offset of the 16-byte word at [t, t + 8) of a row (t a multiple of 8, the row
// 16-byte aligned) to read so that a word past L never leaves the data: it reads the word that
// holds element L - 1 instead. A word that reaches past L is read whole: an aligned 16-byte block
// that holds a valid element lies in that element's page. The elements at or past L are masked
// (mask8) or zeroed in LDS when used, never when loaded, so that every chunk issues the same
// loads and a load never waits for its data where it is issued.
__device__ __forceinline__ int64_t word_at(int64_t t, int64_t L) {
  return t < L ? t : ((L - 1) & ~(int64_t)7);
}
// w with the elements at index >= nv zeroed (nv = valid elements of the word; <= 0: none)
__device__ __forceinline__ u32x4 mask8(const u32x4 w, int nv) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t keep = nv >= 2 * k + 2 ? 0xffffffffu : (nv == 2 * k + 1 ? 0x0000ffffu : 0u);
    r[k] = w[k] & keep;
  }
  return r;
}

// v moved across lanes by the DPP control CTRL in the rows of ROW_MASK; a lane outside those rows,
// or whose source lane lies outside its row, gets 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
// Inclusive prefix sum over the 64 lanes, in registers: shifts right by 1, 2, 4 and 8 lanes
// within each row of 16 lanes (row_shr), then the last lane of rows 0 and 2 is added to rows 1
// and 3 (row_bcast:15), and the last lane of row 1, by then the sum of lanes 0..31, to rows 2
// and 3 (row_bcast:31). Six dependent VALU instructions instead of six LDS round trips.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v += dpp_or_zero<0x111, 0xf>(v);
  v += dpp_or_zero<0x112, 0xf>(v);
  v += dpp_or_zero<0x114, 0xf>(v);
  v += dpp_or_zero<0x118, 0xf>(v);
  v += dpp_or_zero<0x142, 0xa>(v);
  v += dpp_or_zero<0x143, 0xc>(v);
  return v;
}

// Per-chunk step arrays in LDS, kQ floats each: s2 = s_t log2 e, w = w_t, es = e^{s_t},
// cw = e^{s_Q - s_t} w_t.
struct StepArrays {
  float s2[kQ];
  float w[kQ];
  float es[kQ];
  float cw[kQ];
};

// Direct load of 16 bytes per lane from global memory into LDS at lds + 16 * lane (lds is a
// wave-uniform LDS byte address). Written as an instruction of its own rather than the builtin:
// the compiler then keeps no account of it, so it never makes other LDS accesses wait for it (it
// cannot tell which buffer the data go to). The instruction has no register result; the kernel
// waits for it explicitly (vmcnt(0) and a barrier before the buffer is read, and no direct load
// into a buffer is issued before a barrier has ended every read of it). Any wait count that the
// compiler computes for its own loads only over-counts the outstanding operations with these
// present, so it stays correct.
// M0 (the LDS base of the load) is named as clobbered; clang warns that M0 is a reserved
// register, which here only means that nothing else in the kernel may rely on its value across
// the instruction (nothing does: the kernel has no other M0 user).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with vmcnt(0) and the other counters left alone
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// Workgroup barrier for LDS data only: this wavefront's LDS accesses complete, then s_barrier.
// Unlike __syncthreads it does not wait for global memory operations (the next chunk's loads stay
// in flight); the memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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
  constexpr int kTile = N * 128;       // bytes of one staged tile (N rows x 64 bf16)
  constexpr int kLm = kQ * kQ * 2;
  constexpr int kDma = N / 32;         // direct loads per matrix per lane (8 rows per load)
  // two stage buffers of (B tile, C tile, x tile, z tile, delta), Lmat hi and lo parts, step
  // arrays
  constexpr int kXT = kPB * 128;                       // x or z tile: 64 rows of 64 bf16
  constexpr int kOffX = 2 * kTile, kOffZ = kOffX + kXT, kOffD = kOffZ + (GATE ? kXT : 0);
  constexpr int kStage = kOffD + 128;
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t lm_hi[kLm];
  __shared__ __attribute__((aligned(16))) uint8_t lm_lo[kLm];
  __shared__ StepArrays sa[2];
  lds_u8* const lm = (lds_u8*)lm_hi;    // the LDS address space
  lds_u8* const lml = (lds_u8*)lm_lo;

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
  bf16_bits* yrow = Yo + b * p.y_sb + d * p.y_sd;
  const bf16_bits* dlrow = DL + b * p.dl_sb + head * p.dl_sd;
  const float Dp = Dm ? Dm[d] : 0.0f;

  // direct loads: load k of this wavefront fills state rows [8 (4k + wave), +8) of a tile,
  // lane l the 16 bytes at row + l / 8, stored slot l % 8, i.e. logical slot (l % 8) ^ sw(row)
  const int dma_r = lane >> 3;
  const bf16_bits* Bbase = Bm + b * p.B_sb + grp * p.B_sg;
  const bf16_bits* Cbase = Cm + b * p.C_sb + grp * p.C_sg;
  int dma_slot[kDma];
#pragma unroll
  for (int k = 0; k < kDma; ++k) dma_slot[k] = (lane & 7) ^ sw_row(8 * (4 * k + wave) + dma_r);
  // x and z tiles: load k (0, 1) of this wavefront fills channel rows [8 (4k + wave), +8)
  const bf16_bits* xz_row[2];
  const bf16_bits* zz_row[2];
  int xz_slot[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = 8 * (4 * k + wave) + dma_r;
    xz_row[k] = X + b * p.x_sb + (d0 + r) * p.x_sd;
    zz_row[k] = GATE ? Z + b * p.z_sb + (d0 + r) * p.z_sd : nullptr;
    xz_slot[k] = (lane & 7) ^ sw_row(r);
  }

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

  // Direct loads of chunk ch (B, C, x, z) into stage buffer par (= ch & 1, a constant at every
  // call).
  auto issue = [&](int64_t ch, const int par) __attribute__((always_inline)) {
    const int64_t t0 = ch * kQ;
    lds_u8* buf = par ? (lds_u8*)stage1 : (lds_u8*)stage0;
    const uint32_t base = (uint32_t)(uintptr_t)buf;
#pragma unroll
    for (int k = 0; k < kDma; ++k) {
      const int n = 8 * (4 * k + wave) + dma_r;
      const int64_t tw = word_at(t0 + 8 * dma_slot[k], L);
      const uint32_t dst = base + 8 * (4 * k + wave) * 128;  // wave-uniform
      dma16(Bbase + n * p.B_sn + tw, dst);
      dma16(Cbase + n * p.C_sn + tw, dst + kTile);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t tw = word_at(t0 + 8 * xz_slot[k], L);
      const uint32_t dst = base + 8 * (4 * k + wave) * 128;
      dma16(xz_row[k] + tw, dst + kOffX);
      if constexpr (GATE) dma16(zz_row[k] + tw, dst + kOffZ);
    }
  };
  // Direct load of chunk ch's delta (128 bytes, lanes 0..7 of wavefront 3) into the delta slot of
  // stage buffer ch & 1. It runs two chunks ahead, so that the step arrays of chunk ch + 1 can
  // be made while chunk ch computes instead of at the barrier that ends chunk ch.
  auto issue_delta = [&](int64_t ch, const int par) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(uintptr_t)(par ? (lds_u8*)stage1 : (lds_u8*)stage0);
    if (wave == 3 && lane < 8) dma16(dlrow + word_at(ch * kQ + 8 * lane, L), base + kOffD);
  };
  // step arrays of chunk ch (wavefront 2, which has the fewest G^T operands to read), after
  // its loads have landed
  auto steps = [&](int64_t ch, const int par) __attribute__((always_inline)) {
    if (wave == 2) {
      const int64_t t = ch * kQ + lane;
      const bool valid = t < L;
      const lds_u8* buf = par ? (const lds_u8*)stage1 : (const lds_u8*)stage0;
      // steps past L hold other data (a word read in place of one past the end); their
      // results are replaced below
      const bf16_bits raw = *reinterpret_cast<const __attribute__((address_space(3))) bf16_bits*>(
          buf + kOffD + 2 * lane);
      float dl = to_f32(raw) + bias;
      if (softplus) dl = softplus_f32(dl);
      float a2 = dl * a_log2;  // a_t log2 e
      float w = dl;
      if (zoh) w = dl * zoh_ratio(__builtin_amdgcn_exp2f(a2), a2);
      if (!valid) { a2 = 0.0f; w = 0.0f; }
      // a step whose decay 2^a2 is below the smallest fp32 (a2 < -150) zeroes every product
      // through it whatever its exact value, so a2 is clamped at -160: the prefix sums then stay
      // within 64 x 160 of zero, and their differences s_t - s_j keep an absolute error of about
      // 1e-3 even when single steps decay by far more (large delta times large |A|)
      a2 = fmaxf(a2, -160.0f);
      // inclusive prefix sum over the 64 steps of the chunk
      const float s2 = wave_inclusive_sum(a2);
      const float sQ = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s2), 63));
      StepArrays& A = sa[par];
      A.s2[lane] = s2;
      A.w[lane] = w;
      A.es[lane] = __builtin_amdgcn_exp2f(s2);
      A.cw[lane] = __builtin_amdgcn_exp2f(sQ - s2) * w;
    }
  };

  // G^T tile (jt, tt) (jt <= tt): masked, decay-weighted, split and stored into Lmat.
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
      v[q] = (jt < tt || j0 + q <= t) ? acc[q] * __builtin_amdgcn_exp2f(st - sj[q]) * wj[q] : 0.0f;
    const u32x2 s01 = split2(v[0], v[1]), s23 = split2(v[2], v[3]);
    const int o = off_lm(t, 2 * jt + (g >> 1)) + 8 * (g & 1);
    sts8(lm, o, u32x2{s01[0], s23[0]});
    sts8(lml, o, u32x2{s01[1], s23[1]});
  };
  // operands of G^T tile (jt, tt), k-step kk, from the staged tiles: A = B^T rows j, B = C^T
  // rows t; k-slots (g, 0..7) are states 32kk + 8g + (0..7). Lane 4q + r of group g addresses
  // row 32kk + 8g + q (+ 4) at steps 16jt + 4r (+ 0..3).
  const int tr_q = c >> 2, tr_r = c & 3;
  auto g_operand = [&](const lds_u8* tile, int col_tile, int kk) __attribute__((always_inline)) {
    const int n = 32 * kk + 8 * g + tr_q;
    const int slot = 2 * col_tile + (tr_r >> 1);
    const u32x2 lo = ldtr(tile, off_st(n, slot) + 8 * (tr_r & 1));
    const u32x2 hi = ldtr(tile, off_st(n + 4, slot) + 8 * (tr_r & 1));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // G^T tiles that share one operand: with SB the B block S and the C blocks O0, O1, O2, i.e.
  // tiles (S, O_i); otherwise the C block S and the B blocks O_i, tiles (O_i, S). CNT tiles
  // (the first CNT of the O_i). Every argument is a std::integral_constant.
  auto shared_tiles = [&](const StepArrays& A, const lds_u8* bt, const lds_u8* ct, auto sb,
                          auto s_blk, auto cnt, auto o0, auto o1, auto o2)
      __attribute__((always_inline)) {
    constexpr bool SB = decltype(sb)::value;
    constexpr int S = decltype(s_blk)::value, CNT = decltype(cnt)::value;
    constexpr int O[3] = {decltype(o0)::value, decltype(o1)::value, decltype(o2)::value};
    u32x4 sh[NK], ot[CNT][NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      sh[kk] = g_operand(SB ? bt : ct, S, kk);
#pragma unroll
      for (int i = 0; i < CNT; ++i) ot[i][kk] = g_operand(SB ? ct : bt, O[i], kk);
    }
    f32x4 g[CNT];
#pragma unroll
    for (int i = 0; i < CNT; ++i) g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int i = 0; i < CNT; ++i)
        g[i] = SB ? mma(sh[kk], ot[i][kk], g[i]) : mma(ot[i][kk], sh[kk], g[i]);
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) store_lmat(A, SB ? S : O[i], SB ? O[i] : S, g[i]);
  };
  using ic0 = std::integral_constant<int, 0>;
  using ic1 = std::integral_constant<int, 1>;
  using ic2 = std::integral_constant<int, 2>;
  using ic3 = std::integral_constant<int, 3>;
  using kB = std::integral_constant<bool, true>;
  using kC = std::integral_constant<bool, false>;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // chunk ch, par = ch & 1 (a constant at both calls)
  auto chunk = [&](int64_t ch, const int par) __attribute__((always_inline)) {
    lds_u8* const stg = par ? (lds_u8*)stage1 : (lds_u8*)stage0;
    const lds_u8* bt = stg;           // B tile [n][j]
    const lds_u8* ct = stg + kTile;   // C tile [n][t]
    const StepArrays& A = sa[par];
    const int64_t t0 = ch * kQ;
    const bool more = ch + 1 < nchunks;
    if (more) issue(ch + 1, par ^ 1);
    if (ch + 2 < nchunks) issue_delta(ch + 2, par);
    // the step arrays of chunk ch + 1 (its delta landed before the barrier that began chunk ch)
    if (more) steps(ch + 1, par ^ 1);

    // this lane's x and z: steps [16g, 16g + 16) of channel row pl
    u32x4 xv[2], zv[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      xv[s] = lds16(stg + kOffX, off_st(pl, 2 * g + s));
      if constexpr (GATE) zv[s] = lds16(stg + kOffZ, off_st(pl, 2 * g + s));
    }
    if (t0 + kQ > L) {
      // last chunk of a ragged sequence: mask x and z past L
      const int lim = (int)(L - t0);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        xv[s] = mask8(xv[s], lim - (16 * g + 8 * s));
        if constexpr (GATE) zv[s] = mask8(zv[s], lim - (16 * g + 8 * s));
      }
      // and zero the staged B, C words at steps >= L
      lds_u8* w = stg;
      for (int i = tid; i < 2 * N * 8; i += kThreads) {
        const int n = (i >> 3) % N, slot = i & 7;
        const int nv = (int)(L - t0) - 8 * slot;
        if (nv < 8) {
          lds_u8* tile = w + (i >= N * 8 ? kTile : 0);
          sts16(tile, off_st(n, slot), mask8(lds16(tile, off_st(n, slot)), nv));
        }
      }
      sync_lds();
    }

    // 1. Lmat: the wavefront's G^T tiles (see the header comment). The bf16 hi and lo parts of
    //    H that step 2 takes are made in the same block, where they overlap the tiles' products.
    //    k-slots of step kk: states 32kk + 4g + (0..3), then 32kk + 16 + 4g + (0..3)
    u32x4 hb[NK], hl[NK];
    auto split_h = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u32x2 h01 = split2(H[2 * kk][0], H[2 * kk][1]), h23 = split2(H[2 * kk][2], H[2 * kk][3]);
        const u32x2 h45 = split2(H[2 * kk + 1][0], H[2 * kk + 1][1]);
        const u32x2 h67 = split2(H[2 * kk + 1][2], H[2 * kk + 1][3]);
        hb[kk] = u32x4{h01[0], h23[0], h45[0], h67[0]};
        hl[kk] = u32x4{h01[1], h23[1], h45[1], h67[1]};
      }
    };
    if (wv == 0) {
      shared_tiles(A, bt, ct, kB{}, ic0{}, ic3{}, ic0{}, ic1{}, ic2{});
      split_h();
    } else if (wv == 1) {
      shared_tiles(A, bt, ct, kC{}, ic3{}, ic3{}, ic0{}, ic1{}, ic2{});
      split_h();
    } else if (wv == 2) {
      shared_tiles(A, bt, ct, kB{}, ic1{}, ic2{}, ic1{}, ic2{}, ic0{});
      split_h();
    } else {
      shared_tiles(A, bt, ct, kB{}, ic2{}, ic1{}, ic2{}, ic0{}, ic0{});
      shared_tiles(A, bt, ct, kB{}, ic3{}, ic1{}, ic3{}, ic0{}, ic0{});
      split_h();
    }
    sync_lds();

    // 2. Y tiles i = 0..3: row r of tile i is step 16 (r / 4) + 4i + r % 4. First the
    //    inter-chunk part e^{s_t} C^T H, then the intra-chunk part Lmat x. The C^T operand: lane
    //    4q + r of group g addresses state row 32kk + 4g + q (then + 16) at steps 16r + 4i.
    f32x4 Y[4];
    {
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int n = 32 * kk + 4 * g + tr_q;
        u32x4 ca[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 2 * tr_r + (i >> 1);
          const u32x2 lo = ldtr(ct, off_st(n, slot) + 8 * (i & 1));
          const u32x2 hi = ldtr(ct, off_st(n + 16, slot) + 8 * (i & 1));
          ca[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = mma(ca[i], hb[kk], Y[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = mma(ca[i], hl[kk], Y[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[i] *= *reinterpret_cast<const f32x4*>(&A.es[16 * g + 4 * i]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 la[4], ll[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tr = 16 * (c >> 2) + 4 * i + (c & 3);
          la[i] = lds16(lm, off_lm(tr, 2 * g + s));
          ll[i] = lds16(lml, off_lm(tr, 2 * g + s));
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
        for (int m = 0; m < NM; ++m) ba[m] = lds16(bt, off_st(16 * m + c, 2 * g + s));
#pragma unroll
        for (int m = 0; m < NM; ++m) H[m] = mma(ba[m], xs[s], H[m]);
#pragma unroll
        for (int m = 0; m < NM; ++m) H[m] = mma(ba[m], xl[s], H[m]);
      }
    }

    // 5. the next chunk's loads have landed and this chunk's stores have left (every
    //    wavefront waits for its own; on every path, so that no global operation is in
    //    flight where the next chunk begins), then the workgroup moves on
    wait_vmem_all();
    sync_lds();
  };

  issue(0, 0);
  issue_delta(0, 0);
  if (nchunks > 1) issue_delta(1, 1);
  wait_vmem_all();
  __syncthreads();  // wavefront 3's delta loads have landed
  steps(0, 0);
  __syncthreads();
  for (int64_t ch = 0; ch < nchunks; ch += 2) {
    chunk(ch, 0);
    if (ch + 1 >= nchunks) break;
    chunk(ch + 1, 1);
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
