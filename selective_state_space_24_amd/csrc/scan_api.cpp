// C ABI of the selective-scan library: argument validation, segment planning and dispatch.
// Every check runs on the host before anything is enqueued; a failing call launches nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "scan_internal.h"
#include "ssm_scan.h"


namespace {

using ssm::kTargetWaves;
constexpr int64_t kMinSegmentTiles = 8;       // shortest segment worth a summary pass, in tiles
constexpr int64_t kMaxSegments = 65535;       // grid.y limit

struct Plan {
  int64_t nseg;
  int64_t seg_len;
  bool narrow_groups = false;  // bf16 io, 8 < dstate <= 16: 64-channel workgroups (see below)
  bool wave = false;         // bf16 io, 8 < dstate <= 16: the kernel with independent wavefronts
  bool fix = false;          // its split with a zero-start output pass and a correcting pass
};

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Largest element offset + 1 of a (n0, n1, L) tensor with strides (s0, s1, 1); -1 on overflow.
int64_t extent3(int64_t n0, int64_t n1, int64_t L, int64_t s0, int64_t s1) {
  if (n0 == 0 || n1 == 0 || L == 0) return 0;
  int64_t a, b2;
  if (!mul_ok(n0 - 1, s0, &a) || !mul_ok(n1 - 1, s1, &b2)) return -1;
  int64_t e;
  if (__builtin_add_overflow(a, b2, &e) || __builtin_add_overflow(e, L, &e)) return -1;
  return e;
}

int64_t extent4(int64_t n0, int64_t n1, int64_t n2, int64_t L, int64_t s0, int64_t s1, int64_t s2) {
  if (n0 == 0 || n1 == 0 || n2 == 0 || L == 0) return 0;
  int64_t a, b2, c;
  if (!mul_ok(n0 - 1, s0, &a) || !mul_ok(n1 - 1, s1, &b2) || !mul_ok(n2 - 1, s2, &c)) return -1;
  int64_t e;
  if (__builtin_add_overflow(a, b2, &e) || __builtin_add_overflow(e, c, &e) ||
      __builtin_add_overflow(e, L, &e))
    return -1;
  return e;
}

// True when the rows of a tensor with L-contiguous rows, `nd` outer dimensions of sizes n[] and
// element strides s[] (any order), are pairwise disjoint: taken by increasing stride, every
// dimension of size > 1 must step past the whole extent of the dimensions below it.
bool rows_disjoint(int nd, const int64_t* n, const int64_t* s, int64_t L) {
  if (L <= 0) return true;
  int idx[4];
  int k = 0;
  for (int i = 0; i < nd; ++i)
    if (n[i] > 1) idx[k++] = i;
  for (int i = 1; i < k; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && s[idx[j]] < s[idx[j - 1]]; --j) {
      const int t = idx[j]; idx[j] = idx[j - 1]; idx[j - 1] = t;
    }
  int64_t extent = L;
  for (int i = 0; i < k; ++i) {
    const int64_t st = s[idx[i]], cnt = n[idx[i]];
    if (st < extent) return false;
    int64_t e;
    if (!mul_ok(cnt - 1, st, &e) || __builtin_add_overflow(e, extent, &e)) return false;
    extent = e;
  }
  return true;
}

bool rows_disjoint3(int64_t n0, int64_t n1, int64_t L, int64_t s0, int64_t s1) {
  const int64_t n[] = {n0, n1}, s[] = {s0, s1};
  return rows_disjoint(2, n, s, L);
}

// rows of B and C per (batch, group): dstate, or 2 dstate (real, then imaginary parts) with a
// complex A
int64_t bc_rows(const ssm_scan_desc* d) {
  return d->a_mode == SSM_A_COMPLEX ? 2 * d->dstate : d->dstate;
}

int check_desc(const ssm_scan_desc* d) {
  if (!d) return SSM_ERR_NULL_ARG;
  if (d->io_dtype != SSM_DTYPE_F32 && d->io_dtype != SSM_DTYPE_BF16) return SSM_ERR_BAD_DTYPE;
  if (d->a_mode != SSM_A_DIAG && d->a_mode != SSM_A_HEAD && d->a_mode != SSM_A_COMPLEX)
    return SSM_ERR_BAD_DTYPE;
  if (d->batch < 0 || d->seqlen < 0 || d->dim < 1 || d->dstate < 1 || d->dstate > SSM_MAX_DSTATE ||
      d->ngroups < 1 || d->headdim < 1)
    return SSM_ERR_BAD_SHAPE;
  if (d->dim % d->ngroups || d->dim % d->headdim) return SSM_ERR_BAD_SHAPE;
  if (d->a_mode != SSM_A_HEAD && d->headdim != 1) return SSM_ERR_BAD_SHAPE;
  int64_t t;
  if (!mul_ok(d->batch, d->dim, &t) || !mul_ok(t, d->seqlen, &t) || !mul_ok(t, d->dstate, &t))
    return SSM_ERR_BAD_SHAPE;
  const int64_t strides[] = {d->x_stride_batch, d->x_stride_dim, d->delta_stride_batch,
                             d->delta_stride_dim, d->B_stride_batch, d->B_stride_group,
                             d->B_stride_state, d->C_stride_batch, d->C_stride_group,
                             d->C_stride_state, d->z_stride_batch, d->z_stride_dim,
                             d->y_stride_batch, d->y_stride_dim};
  for (int64_t s : strides)
    if (s < 0) return SSM_ERR_BAD_STRIDE;
  // y rows must be disjoint (they are written)
  if (!rows_disjoint3(d->batch, d->dim, d->seqlen, d->y_stride_batch, d->y_stride_dim))
    return SSM_ERR_BAD_STRIDE;
  const int64_t drows = d->a_mode == SSM_A_HEAD ? d->dim / d->headdim : d->dim;
  if (extent3(d->batch, d->dim, d->seqlen, d->x_stride_batch, d->x_stride_dim) < 0 ||
      extent3(d->batch, drows, d->seqlen, d->delta_stride_batch, d->delta_stride_dim) < 0 ||
      extent3(d->batch, d->dim, d->seqlen, d->z_stride_batch, d->z_stride_dim) < 0 ||
      extent3(d->batch, d->dim, d->seqlen, d->y_stride_batch, d->y_stride_dim) < 0 ||
      extent4(d->batch, d->ngroups, bc_rows(d), d->seqlen, d->B_stride_batch, d->B_stride_group,
              d->B_stride_state) < 0 ||
      extent4(d->batch, d->ngroups, bc_rows(d), d->seqlen, d->C_stride_batch, d->C_stride_group,
              d->C_stride_state) < 0)
    return SSM_ERR_BAD_SHAPE;
  return SSM_OK;
}

Plan plan_segments(const ssm_scan_desc* d) {
  const int64_t tile = ssm::kLT;
  const int64_t cpg = ssm::kChannelsPerGroup;
  const int64_t groups = d->batch * ((d->dim + cpg - 1) / cpg);
  const int64_t waves = groups * ssm::kWavesPerGroup;
  Plan p{1, d->seqlen > 0 ? d->seqlen : 1};
  if (groups == 0 || d->seqlen == 0) return p;
  if (ssm::groups_fill_chip(groups)) return p;  // enough channel groups: one pass
  int64_t want = (kTargetWaves + waves - 1) / waves;
  if (d->io_dtype == SSM_DTYPE_BF16 && d->dstate > 8 && d->dstate <= 16) {
    // bf16 io with 8 < N <= 16 runs the kernel with independent wavefronts, one 8-wavefront
    // workgroup (128 channels) per CU, except where narrow_one_pass holds: then 64-channel
    // workgroups of four wavefronts spread over more CUs and need no summary pass (measured
    // 163 us per-step median; the barrier-synchronised kernel with eight wavefronts of two
    // states 167 us, with four of four 183 us, against 192-204 us split along L, at batch 8,
    // d_inner 1536, L 2048)
    if (ssm::narrow_one_pass(groups)) {
      p.narrow_groups = true;
      return p;
    }
    p.wave = true;
    // otherwise segments: beyond what fills the chip once they would start a second round of
    // workgroups that leaves most CUs idle, so the count is rounded down
    want = kTargetWaves / waves;
  }
  const int64_t tiles = (d->seqlen + tile - 1) / tile;
  const int64_t max_by_len = tiles / kMinSegmentTiles;
  if (want > max_by_len) want = max_by_len;
  if (want > kMaxSegments) want = kMaxSegments;
  if (want <= 1) return p;
  const int64_t seg_tiles = (tiles + want - 1) / want;
  p.seg_len = seg_tiles * tile;
  p.nseg = (d->seqlen + p.seg_len - 1) / p.seg_len;
  if (p.nseg <= 1) p = Plan{1, d->seqlen};
  // long segments: zero-start output pass and correcting pass (see scan_fwd_wave_kernel)
  p.fix = p.wave && p.nseg > 1 && p.seg_len >= ssm::kFixMinSegment;
  return p;
}

// States the split output pass of the independent-wavefront kernel stores per segment for the
// correcting pass: one per kFixCheck steps, at most kFixMaxChecks (0 when `checks` is off).
int64_t fix_checks(const Plan& p, bool checks) {
  if (!checks || !p.fix) return 0;
  return std::min<int64_t>(p.seg_len / ssm::kFixCheck, ssm::kFixMaxChecks);
}

// Workspace of a split sequence: hend (batch, dim, nseg, N) fp32, then dsum (batch, dim, nseg)
// fp32, then (the correcting scheme) the stored states (batch, dim, nseg, nchk, 16) fp32, from
// the next 16-byte boundary (12 bytes of slack allow for a 4-byte-aligned base).
size_t workspace_bytes_for(const ssm_scan_desc* d, const Plan& p, bool checks = true) {
  if (p.nseg <= 1) return 0;
  const size_t bdn = (size_t)d->batch * (size_t)d->dim * (size_t)p.nseg;
  size_t bytes = bdn * (size_t)(d->dstate + 1) * sizeof(float);
  const int64_t nchk = fix_checks(p, checks);
  if (nchk > 0) bytes += 12 + bdn * (size_t)nchk * 16 * sizeof(float);
  return bytes;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of the backward pass: checkpoints (batch, ntiles, N, dim) every kCkptStep steps, the
// dB and dC partials (batch, groups_per_batch, N, L), the dA partials (batch, dim, N), dD and
// dbias partials (batch, dim); in head mode also ddelta summed over runs of gcd(headdim, 64)
// channels (batch, dim / span, L) and the bias-gradient partials (nheads, batch, chunks). fp32,
// each section 256-byte aligned.
struct BwdLayout {
  size_t ckpt, dB, dC, dA, dD, dbias, ddl, dbh, total;
  int64_t span;
};

int64_t gcd64(int64_t a, int64_t b) {
  while (b) { const int64_t t = a % b; a = b; b = t; }
  return a;
}

BwdLayout bwd_layout(const ssm_scan_desc* d) {
  const size_t ntiles = (size_t)((d->seqlen + ssm::kCkptStep - 1) / ssm::kCkptStep);
  const size_t gpb = (size_t)((d->dim + ssm::kChannelsPerGroup - 1) / ssm::kChannelsPerGroup);
  const size_t B = (size_t)d->batch, D = (size_t)d->dim, N = (size_t)d->dstate, L = (size_t)d->seqlen;
  const bool head = d->a_mode == SSM_A_HEAD;
  BwdLayout l;
  l.span = head ? gcd64(d->headdim, ssm::kChannelsPerGroup) : 1;
  size_t off = 0;
  l.ckpt = off; off += align256(B * D * ntiles * N * 4);
  l.dB = off; off += align256(B * gpb * N * L * 4);
  l.dC = off; off += align256(B * gpb * N * L * 4);
  l.dA = off; off += align256(B * D * N * 4);
  l.dD = off; off += align256(B * D * 4);
  l.dbias = off; off += align256(B * D * 4);
  l.ddl = off;
  if (head) off += align256(B * (D / (size_t)l.span) * L * 4);
  l.dbh = off;
  if (head) {
    const size_t chunks = (L + ssm::kHeadDeltaChunk - 1) / ssm::kHeadDeltaChunk;
    off += align256((D / (size_t)d->headdim) * B * chunks * 4);
  }
  l.total = (B == 0 || L == 0) ? 0 : off;
  return l;
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b || abytes == 0 || bbytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The forward scan with a complex diagonal A (a_mode SSM_A_COMPLEX), after check_desc: the
// delta * B rule, no initial or final state, the recurrent algorithm, dstate <= 32.
int complex_fwd(const ssm_scan_desc& d, const void* x, const void* delta, const float* A,
                const void* B, const void* C, const float* D, const void* z,
                const float* delta_bias, int32_t delta_softplus, void* y, int32_t disc,
                int32_t algo, const float* h0, const float* hfin, void* stream) {
  if (disc != SSM_DISC_DELTA_B || algo == SSM_ALGO_CHUNKED || h0 || hfin ||
      d.dstate > SSM_MAX_COMPLEX_DSTATE)
    return SSM_ERR_UNSUPPORTED;
  // the B and C of a workgroup's 64 channels come from one group
  if (d.ngroups > 1 && (d.dim / d.ngroups) % ssm::kChannelsPerGroup != 0)
    return SSM_ERR_UNSUPPORTED;
  if (d.batch == 0 || d.seqlen == 0) return SSM_OK;
  if (!x || !delta || !A || !B || !C || !y) return SSM_ERR_NULL_ARG;
  const bool bf16 = d.io_dtype == SSM_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  const void* io_ptrs[] = {x, delta, B, C, z, y};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_MISALIGNED;
  const void* f32_ptrs[] = {A, D, delta_bias};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_MISALIGNED;
  const size_t y_bytes =
      (size_t)extent3(d.batch, d.dim, d.seqlen, d.y_stride_batch, d.y_stride_dim) * es;
  const size_t in_bytes[] = {
      (size_t)extent3(d.batch, d.dim, d.seqlen, d.x_stride_batch, d.x_stride_dim) * es,
      (size_t)extent3(d.batch, d.dim, d.seqlen, d.delta_stride_batch, d.delta_stride_dim) * es,
      (size_t)extent4(d.batch, d.ngroups, 2 * d.dstate, d.seqlen, d.B_stride_batch,
                      d.B_stride_group, d.B_stride_state) * es,
      (size_t)extent4(d.batch, d.ngroups, 2 * d.dstate, d.seqlen, d.C_stride_batch,
                      d.C_stride_group, d.C_stride_state) * es,
      z ? (size_t)extent3(d.batch, d.dim, d.seqlen, d.z_stride_batch, d.z_stride_dim) * es : 0,
      (size_t)d.dim * d.dstate * 2 * 4,
      D ? (size_t)d.dim * 4 : 0,
      delta_bias ? (size_t)d.dim * 4 : 0};
  const void* in_ptrs[] = {x, delta, B, C, z, A, D, delta_bias};
  for (int i = 0; i < 8; ++i)
    if (overlaps(y, y_bytes, in_ptrs[i], in_bytes[i])) return SSM_ERR_ALIAS;

  ssm::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.delta_bias = delta_bias;
  p.y = y;
  p.batch = d.batch; p.dim = d.dim; p.L = d.seqlen; p.N = d.dstate; p.ngroups = d.ngroups;
  p.headdim = 1;
  p.x_sb = d.x_stride_batch; p.x_sd = d.x_stride_dim;
  p.dl_sb = d.delta_stride_batch; p.dl_sd = d.delta_stride_dim;
  p.B_sb = d.B_stride_batch; p.B_sg = d.B_stride_group; p.B_sn = d.B_stride_state;
  p.C_sb = d.C_stride_batch; p.C_sg = d.C_stride_group; p.C_sn = d.C_stride_state;
  p.z_sb = d.z_stride_batch; p.z_sd = d.z_stride_dim;
  p.y_sb = d.y_stride_batch; p.y_sd = d.y_stride_dim;
  p.softplus = delta_softplus ? 1 : 0;
  // 16-byte row access of x, delta, z, y: aligned bases, strides multiples of 16 bytes
  const int64_t vec = 16 / (int64_t)es;
  bool vec_ok = true;
  const void* vptrs[] = {x, delta, z, y};
  for (const void* q : vptrs)
    if (q && !aligned(q, 16)) vec_ok = false;
  for (int64_t st : {d.x_stride_batch, d.x_stride_dim, d.delta_stride_batch, d.delta_stride_dim,
                     z ? d.z_stride_batch : 0, z ? d.z_stride_dim : 0, d.y_stride_batch,
                     d.y_stride_dim})
    if (st % vec) vec_ok = false;
  p.vec_io = vec_ok ? 1 : 0;
  bool bc_ok = aligned(B, 16) && aligned(C, 16);
  for (int64_t st : {d.B_stride_batch, d.B_stride_group, d.B_stride_state, d.C_stride_batch,
                     d.C_stride_group, d.C_stride_state})
    if (st % vec) bc_ok = false;
  p.bc_vec = bc_ok ? 1 : 0;
  const hipError_t e = ssm::launch_complex(p, bf16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

int ssm_wave_simd_ids(int32_t* out, int32_t nworkgroups, void* stream) {
  if (!out) return SSM_ERR_NULL_ARG;
  if (nworkgroups < 0) return SSM_ERR_BAD_SHAPE;
  const hipError_t e = ssm::launch_wave_simd(out, nworkgroups, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case SSM_ERR_BAD_SHAPE: return "invalid sizes (negative, zero where >= 1 is needed, indivisible dim, dstate > 128, or overflow)";
    case SSM_ERR_BAD_DTYPE: return "unknown io dtype or A mode";
    case SSM_ERR_BAD_STRIDE: return "invalid strides (negative, or overlapping output rows)";
    case SSM_ERR_MISALIGNED: return "a pointer is not aligned to its element size";
    case SSM_ERR_ALIAS: return "the output overlaps an input";
    case SSM_ERR_WORKSPACE: return "workspace missing or smaller than the queried size";
    case SSM_ERR_HIP: return "the HIP runtime reported an error";
    case SSM_ERR_UNSUPPORTED: return "valid arguments outside what this build implements";
    case SSM_ERR_SCRATCH_LIMIT: return "the problem needs more scratch than the fixed array of the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int ssm_scan_desc_init_contiguous(ssm_scan_desc* d, int64_t batch, int64_t dim, int64_t seqlen,
                                  int64_t dstate, int64_t ngroups, int64_t headdim,
                                  int32_t io_dtype, int32_t a_mode) {
  if (!d) return SSM_ERR_NULL_ARG;
  memset(d, 0, sizeof(*d));
  d->batch = batch; d->dim = dim; d->seqlen = seqlen; d->dstate = dstate;
  d->ngroups = ngroups; d->headdim = headdim; d->io_dtype = io_dtype; d->a_mode = a_mode;
  const int64_t rows = (a_mode == SSM_A_HEAD && headdim > 0) ? dim / headdim : dim;
  d->x_stride_dim = seqlen; d->x_stride_batch = dim * seqlen;
  d->delta_stride_dim = seqlen; d->delta_stride_batch = rows * seqlen;
  const int64_t bc = a_mode == SSM_A_COMPLEX ? 2 * dstate : dstate;  // B/C rows per group
  d->B_stride_state = seqlen; d->B_stride_group = bc * seqlen; d->B_stride_batch = ngroups * bc * seqlen;
  d->C_stride_state = d->B_stride_state; d->C_stride_group = d->B_stride_group; d->C_stride_batch = d->B_stride_batch;
  d->z_stride_dim = seqlen; d->z_stride_batch = dim * seqlen;
  d->y_stride_dim = seqlen; d->y_stride_batch = dim * seqlen;
  return SSM_OK;
}

int ssm_selective_scan_workspace_size(const ssm_scan_desc* desc, size_t* bytes) {
  if (!bytes) return SSM_ERR_NULL_ARG;
  const int rc = check_desc(desc);
  if (rc != SSM_OK) return rc;
  *bytes = ssm::fwd_workspace_bytes(desc, true);
  return SSM_OK;
}

}  // extern "C"

namespace ssm {

size_t fwd_workspace_bytes(const ssm_scan_desc* desc, bool checks) {
  // the complex-A scan runs in one pass without workspace
  return desc->a_mode == SSM_A_COMPLEX ? 0 : workspace_bytes_for(desc, plan_segments(desc), checks);
}

int fwd_ext(const ssm_scan_desc* desc, const void* x, const void* delta, const float* A,
            const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
            int32_t delta_softplus, void* y, const ssm_scan_ext* ext, void* workspace,
            size_t workspace_bytes, void* stream, bool checks) {
  int rc = check_desc(desc);
  if (rc != SSM_OK) return rc;
  const int32_t disc = ext ? ext->discretization : SSM_DISC_DELTA_B;
  if (disc != SSM_DISC_DELTA_B && disc != SSM_DISC_ZOH) return SSM_ERR_BAD_DTYPE;
  const int32_t algo = ext ? ext->algorithm : SSM_ALGO_AUTO;
  if (algo != SSM_ALGO_AUTO && algo != SSM_ALGO_RECURRENT && algo != SSM_ALGO_CHUNKED)
    return SSM_ERR_BAD_DTYPE;
  const float* h0 = ext ? ext->h0 : nullptr;
  float* hfin = ext ? ext->h_final : nullptr;
  const ssm_scan_desc& d = *desc;
  if (d.a_mode == SSM_A_COMPLEX)
    return complex_fwd(d, x, delta, A, B, C, D, z, delta_bias, delta_softplus, y, disc, algo, h0,
                       hfin, stream);
  if (d.batch == 0) return SSM_OK;  // nothing to compute or write
  if (d.seqlen == 0) {
    // no steps: the final state is the initial one (zero without h0)
    if (!hfin) return SSM_OK;
    const size_t sbytes = (size_t)d.batch * d.dim * d.dstate * sizeof(float);
    if (!aligned(hfin, 4) || (h0 && !aligned(h0, 4))) return SSM_ERR_MISALIGNED;
    if (h0 && overlaps(hfin, sbytes, h0, sbytes)) return SSM_ERR_ALIAS;
    const hipError_t e = ssm::launch_state_copy(h0, hfin, (int64_t)(sbytes / sizeof(float)),
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  if (!x || !delta || !A || !B || !C || !y) return SSM_ERR_NULL_ARG;

  const bool bf16 = d.io_dtype == SSM_DTYPE_BF16;
  const bool head = d.a_mode == SSM_A_HEAD;
  const size_t es = bf16 ? 2 : 4;
  const int64_t nheads = d.dim / d.headdim;
  const int64_t drows = head ? nheads : d.dim;
  const void* io_ptrs[] = {x, delta, B, C, z, y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_MISALIGNED;
  const void* f32_ptrs[] = {A, D, delta_bias, h0, hfin};
  for (const void* p : f32_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;

  // outputs (y, the final state, the workspace) must not overlap any input or each other
  const size_t y_bytes = (size_t)extent3(d.batch, d.dim, d.seqlen, d.y_stride_batch, d.y_stride_dim) * es;
  const size_t state_bytes = (size_t)d.batch * d.dim * d.dstate * sizeof(float);
  const size_t in_bytes[] = {
      (size_t)extent3(d.batch, d.dim, d.seqlen, d.x_stride_batch, d.x_stride_dim) * es,
      (size_t)extent3(d.batch, drows, d.seqlen, d.delta_stride_batch, d.delta_stride_dim) * es,
      (size_t)extent4(d.batch, d.ngroups, d.dstate, d.seqlen, d.B_stride_batch, d.B_stride_group, d.B_stride_state) * es,
      (size_t)extent4(d.batch, d.ngroups, d.dstate, d.seqlen, d.C_stride_batch, d.C_stride_group, d.C_stride_state) * es,
      z ? (size_t)extent3(d.batch, d.dim, d.seqlen, d.z_stride_batch, d.z_stride_dim) * es : 0,
      (size_t)(head ? nheads : d.dim * d.dstate) * 4,
      D ? (size_t)d.dim * 4 : 0,
      delta_bias ? (size_t)drows * 4 : 0,
      h0 ? state_bytes : 0};
  const void* in_ptrs[] = {x, delta, B, C, z, A, D, delta_bias, h0};
  constexpr int kInputs = 9;
  for (int i = 0; i < kInputs; ++i) {
    if (overlaps(y, y_bytes, in_ptrs[i], in_bytes[i])) return SSM_ERR_ALIAS;
    if (hfin && overlaps(hfin, state_bytes, in_ptrs[i], in_bytes[i])) return SSM_ERR_ALIAS;
  }
  if (hfin && overlaps(hfin, state_bytes, y, y_bytes)) return SSM_ERR_ALIAS;

  // B and C must be uniform over each workgroup's channels
  const int64_t ch_per_group = d.dim / d.ngroups;
  if (d.ngroups > 1 && ch_per_group % ssm::kChannelsPerGroup != 0) return SSM_ERR_UNSUPPORTED;

  const Plan plan = plan_segments(desc);

  ssm::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.delta_bias = delta_bias;
  p.y = y; p.h0 = h0; p.hfin = hfin;
  p.batch = d.batch; p.dim = d.dim; p.L = d.seqlen; p.N = d.dstate; p.ngroups = d.ngroups;
  p.headdim = d.headdim;
  p.x_sb = d.x_stride_batch; p.x_sd = d.x_stride_dim;
  p.dl_sb = d.delta_stride_batch; p.dl_sd = d.delta_stride_dim;
  p.B_sb = d.B_stride_batch; p.B_sg = d.B_stride_group; p.B_sn = d.B_stride_state;
  p.C_sb = d.C_stride_batch; p.C_sg = d.C_stride_group; p.C_sn = d.C_stride_state;
  p.z_sb = d.z_stride_batch; p.z_sd = d.z_stride_dim;
  p.y_sb = d.y_stride_batch; p.y_sd = d.y_stride_dim;
  p.groups_per_batch = (d.dim + ssm::kChannelsPerGroup - 1) / ssm::kChannelsPerGroup;
  p.seg_len = plan.seg_len;
  p.nseg = (int32_t)plan.nseg;
  p.narrow_groups = plan.narrow_groups ? 1 : 0;
  p.fix_split = plan.fix ? 1 : 0;
  p.softplus = delta_softplus ? 1 : 0;
  p.zoh = disc == SSM_DISC_ZOH ? 1 : 0;
  // 16-byte vector access of x/delta/z/y rows: 16-byte aligned bases, strides multiple of 16 B
  const int64_t vec = 16 / (int64_t)es;
  bool vec_ok = true;
  const void* vptrs[] = {x, delta, z, y};
  for (const void* q : vptrs)
    if (q && !aligned(q, 16)) vec_ok = false;
  const int64_t vstrides[] = {d.x_stride_batch, d.x_stride_dim, d.delta_stride_batch,
                              d.delta_stride_dim, z ? d.z_stride_batch : 0, z ? d.z_stride_dim : 0,
                              d.y_stride_batch, d.y_stride_dim};
  for (int64_t st : vstrides)
    if (st % vec) vec_ok = false;
  p.vec_io = vec_ok ? 1 : 0;
  bool bc_vec = aligned(B, 16) && aligned(C, 16);
  const int64_t bstrides[] = {d.B_stride_batch, d.B_stride_group, d.B_stride_state,
                              d.C_stride_batch, d.C_stride_group, d.C_stride_state};
  for (int64_t st : bstrides)
    if (st % vec) bc_vec = false;
  p.bc_vec = bc_vec ? 1 : 0;
  const hipStream_t hs = static_cast<hipStream_t>(stream);

  // the chunked form: bf16 io, one A per head, 16-byte access everywhere (states included)
  const bool chunked_ok = bf16 && head && ssm::ssd_supported(p) && (!h0 || aligned(h0, 16)) &&
                          (!hfin || aligned(hfin, 16));
  if (algo == SSM_ALGO_CHUNKED && !chunked_ok) return SSM_ERR_UNSUPPORTED;
  if (algo != SSM_ALGO_RECURRENT && chunked_ok) {
    const hipError_t e = ssm::launch_ssd(p, hs);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }

  const size_t need = workspace_bytes_for(desc, plan, checks);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSM_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 4)) return SSM_ERR_MISALIGNED;
  if (need > 0) {
    for (int i = 0; i < kInputs; ++i)
      if (overlaps(workspace, need, in_ptrs[i], in_bytes[i])) return SSM_ERR_ALIAS;
    if (overlaps(workspace, need, y, y_bytes)) return SSM_ERR_ALIAS;
    if (hfin && overlaps(workspace, need, hfin, state_bytes)) return SSM_ERR_ALIAS;
  }
  if (plan.nseg > 1) {
    const size_t bdn = (size_t)d.batch * d.dim * plan.nseg;
    p.hend = static_cast<float*>(workspace);
    p.dsum = p.hend + bdn * d.dstate;
    p.nchk = fix_checks(plan, checks);
    if (p.nchk > 0)
      p.hchk = reinterpret_cast<float*>(((uintptr_t)(p.dsum + bdn) + 15) & ~(uintptr_t)15);
  }

  hipError_t e;
  if (bf16) e = head ? ssm::launch_bf16_head(p, hs) : ssm::launch_bf16_diag(p, hs);
  else e = head ? ssm::launch_f32_head(p, hs) : ssm::launch_f32_diag(p, hs);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm

extern "C" {

int ssm_selective_scan_fwd_ext(const ssm_scan_desc* desc, const void* x, const void* delta,
                               const float* A, const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, int32_t delta_softplus,
                               void* y, const ssm_scan_ext* ext, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return ssm::fwd_ext(desc, x, delta, A, B, C, D, z, delta_bias, delta_softplus, y, ext,
                      workspace, workspace_bytes, stream, true);
}

int ssm_selective_scan_fwd(const ssm_scan_desc* desc, const void* x, const void* delta,
                           const float* A, const void* B, const void* C, const float* D,
                           const void* z, const float* delta_bias, int32_t delta_softplus,
                           void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return ssm_selective_scan_fwd_ext(desc, x, delta, A, B, C, D, z, delta_bias, delta_softplus, y,
                                    nullptr, workspace, workspace_bytes, stream);
}

int ssm_selective_state_update(const ssm_scan_desc* desc, float* state, const void* x,
                               const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias,
                               int32_t delta_softplus, void* y, void* stream) {
  int rc = check_desc(desc);
  if (rc != SSM_OK) return rc;
  const ssm_scan_desc& d = *desc;
  if (d.a_mode == SSM_A_COMPLEX) return SSM_ERR_UNSUPPORTED;
  if (d.seqlen != 1) return SSM_ERR_BAD_SHAPE;
  if (d.batch == 0) return SSM_OK;
  if (!state || !x || !delta || !A || !B || !C || !y) return SSM_ERR_NULL_ARG;

  const bool bf16 = d.io_dtype == SSM_DTYPE_BF16;
  const bool head = d.a_mode == SSM_A_HEAD;
  const size_t es = bf16 ? 2 : 4;
  const int64_t nheads = d.dim / d.headdim;
  const int64_t drows = head ? nheads : d.dim;
  const void* io_ptrs[] = {x, delta, B, C, z, y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_MISALIGNED;
  const void* f32_ptrs[] = {A, D, delta_bias, state};
  for (const void* p : f32_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;

  const size_t y_bytes = (size_t)extent3(d.batch, d.dim, 1, d.y_stride_batch, d.y_stride_dim) * es;
  const size_t state_bytes = (size_t)d.batch * d.dim * d.dstate * sizeof(float);
  const size_t in_bytes[] = {
      (size_t)extent3(d.batch, d.dim, 1, d.x_stride_batch, d.x_stride_dim) * es,
      (size_t)extent3(d.batch, drows, 1, d.delta_stride_batch, d.delta_stride_dim) * es,
      (size_t)extent4(d.batch, d.ngroups, d.dstate, 1, d.B_stride_batch, d.B_stride_group, d.B_stride_state) * es,
      (size_t)extent4(d.batch, d.ngroups, d.dstate, 1, d.C_stride_batch, d.C_stride_group, d.C_stride_state) * es,
      z ? (size_t)extent3(d.batch, d.dim, 1, d.z_stride_batch, d.z_stride_dim) * es : 0,
      (size_t)(head ? nheads : d.dim * d.dstate) * 4,
      D ? (size_t)d.dim * 4 : 0,
      delta_bias ? (size_t)drows * 4 : 0};
  const void* in_ptrs[] = {x, delta, B, C, z, A, D, delta_bias};
  for (int i = 0; i < 8; ++i) {
    if (overlaps(y, y_bytes, in_ptrs[i], in_bytes[i])) return SSM_ERR_ALIAS;
    if (overlaps(state, state_bytes, in_ptrs[i], in_bytes[i])) return SSM_ERR_ALIAS;
  }
  if (overlaps(state, state_bytes, y, y_bytes)) return SSM_ERR_ALIAS;

  ssm::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.delta_bias = delta_bias;
  p.y = y; p.h0 = state; p.hfin = state;
  p.batch = d.batch; p.dim = d.dim; p.L = 1; p.N = d.dstate; p.ngroups = d.ngroups;
  p.headdim = d.headdim;
  p.x_sb = d.x_stride_batch; p.x_sd = d.x_stride_dim;
  p.dl_sb = d.delta_stride_batch; p.dl_sd = d.delta_stride_dim;
  p.B_sb = d.B_stride_batch; p.B_sg = d.B_stride_group; p.B_sn = d.B_stride_state;
  p.C_sb = d.C_stride_batch; p.C_sg = d.C_stride_group; p.C_sn = d.C_stride_state;
  p.z_sb = d.z_stride_batch; p.z_sd = d.z_stride_dim;
  p.y_sb = d.y_stride_batch; p.y_sd = d.y_stride_dim;
  p.softplus = delta_softplus ? 1 : 0;
  p.state_vec = (d.dstate % 4 == 0 && aligned(state, 16)) ? 1 : 0;
  p.a_vec = (!head && d.dstate % 4 == 0 && aligned(A, 16)) ? 1 : 0;
  // 4 consecutive states of B and C in one 8- (bf16) or 16-byte (fp32) load
  const bool bc4 = d.B_stride_state == 1 && d.C_stride_state == 1 && d.dstate % 4 == 0 &&
                   d.B_stride_batch % 4 == 0 && d.B_stride_group % 4 == 0 &&
                   d.C_stride_batch % 4 == 0 && d.C_stride_group % 4 == 0 &&
                   aligned(B, 4 * es) && aligned(C, 4 * es);
  p.bc_vec = bc4 ? 1 : 0;
  const hipError_t e = ssm::launch_decode(p, bf16, head, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_selective_scan_bwd_workspace_size(const ssm_scan_desc* desc, size_t* bytes) {
  if (!bytes) return SSM_ERR_NULL_ARG;
  const int rc = check_desc(desc);
  if (rc != SSM_OK) return rc;
  if (desc->a_mode == SSM_A_COMPLEX) return SSM_ERR_UNSUPPORTED;
  *bytes = bwd_layout(desc).total;
  return SSM_OK;
}

int ssm_selective_scan_bwd_ext(const ssm_scan_desc* desc, const void* x, const void* delta,
                               const float* A, const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, int32_t delta_softplus,
                               const float* h0, const void* dy, void* dx, void* ddelta,
                               float* dA, float* dB, float* dC, float* dD, void* dz,
                               float* ddelta_bias, float* dh0, const ssm_bwd_ext* ext,
                               void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc != SSM_OK) return rc;
  const ssm_scan_desc& d = *desc;
  if (d.a_mode == SSM_A_COMPLEX) return SSM_ERR_UNSUPPORTED;
  const int32_t disc = ext ? ext->discretization : SSM_DISC_DELTA_B;
  if (disc != SSM_DISC_DELTA_B && disc != SSM_DISC_ZOH) return SSM_ERR_BAD_DTYPE;
  const float* dhfin = ext ? ext->dh_final : nullptr;
  const bool head = d.a_mode == SSM_A_HEAD;
  const int64_t ch_per_group = d.dim / d.ngroups;
  if (d.ngroups > 1 && ch_per_group % ssm::kChannelsPerGroup != 0) return SSM_ERR_UNSUPPORTED;
  if (!dA) return SSM_ERR_NULL_ARG;
  if (z && !dz) return SSM_ERR_NULL_ARG;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t es = d.io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const int64_t nheads = d.dim / d.headdim;
  const int64_t drows = head ? nheads : d.dim;
  const int64_t a_count = head ? nheads : d.dim * d.dstate;
  const size_t a_bytes = (size_t)a_count * 4;
  const size_t state_bytes = (size_t)d.batch * d.dim * d.dstate * 4;
  if (d.batch == 0 || d.seqlen == 0) {
    // nothing depends on the parameters; the initial state's gradient is the final state's
    if (!aligned(dA, 4) || (dD && !aligned(dD, 4)) || (ddelta_bias && !aligned(ddelta_bias, 4)) ||
        (dh0 && !aligned(dh0, 4)) || (dhfin && !aligned(dhfin, 4)))
      return SSM_ERR_MISALIGNED;
    if (dh0 && dhfin && overlaps(dh0, state_bytes, dhfin, state_bytes)) return SSM_ERR_ALIAS;
    hipError_t e = ssm::launch_state_copy(nullptr, dA, a_count, hs);
    if (e == hipSuccess && dD) e = ssm::launch_state_copy(nullptr, dD, d.dim, hs);
    if (e == hipSuccess && ddelta_bias) e = ssm::launch_state_copy(nullptr, ddelta_bias, drows, hs);
    if (e == hipSuccess && dh0) e = ssm::launch_state_copy(dhfin, dh0, (int64_t)(state_bytes / 4), hs);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dB || !dC) return SSM_ERR_NULL_ARG;
  // dx, ddelta, dz, dB and dC are written with the strides of x, delta, z, B and C: inputs may
  // overlap themselves (a broadcast B, say), gradients may not
  {
    const int64_t nbc[] = {d.batch, d.ngroups, d.dstate};
    const int64_t sB[] = {d.B_stride_batch, d.B_stride_group, d.B_stride_state};
    const int64_t sC[] = {d.C_stride_batch, d.C_stride_group, d.C_stride_state};
    if (!rows_disjoint3(d.batch, d.dim, d.seqlen, d.x_stride_batch, d.x_stride_dim) ||
        !rows_disjoint3(d.batch, drows, d.seqlen, d.delta_stride_batch, d.delta_stride_dim) ||
        (z && !rows_disjoint3(d.batch, d.dim, d.seqlen, d.z_stride_batch, d.z_stride_dim)) ||
        !rows_disjoint(3, nbc, sB, d.seqlen) || !rows_disjoint(3, nbc, sC, d.seqlen))
      return SSM_ERR_BAD_STRIDE;
  }

  const void* io_ptrs[] = {x, delta, B, C, z, dy, dx, ddelta, dz};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_MISALIGNED;
  const void* f32_ptrs[] = {A, D, delta_bias, h0, dA, dB, dC, dD, ddelta_bias, dh0, dhfin, workspace};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_MISALIGNED;

  const size_t x_bytes = (size_t)extent3(d.batch, d.dim, d.seqlen, d.x_stride_batch, d.x_stride_dim) * es;
  const size_t dl_bytes = (size_t)extent3(d.batch, drows, d.seqlen, d.delta_stride_batch, d.delta_stride_dim) * es;
  const size_t z_bytes = (size_t)extent3(d.batch, d.dim, d.seqlen, d.z_stride_batch, d.z_stride_dim) * es;
  const size_t y_bytes = (size_t)extent3(d.batch, d.dim, d.seqlen, d.y_stride_batch, d.y_stride_dim) * es;
  const int64_t Bext = extent4(d.batch, d.ngroups, d.dstate, d.seqlen, d.B_stride_batch, d.B_stride_group, d.B_stride_state);
  const int64_t Cext = extent4(d.batch, d.ngroups, d.dstate, d.seqlen, d.C_stride_batch, d.C_stride_group, d.C_stride_state);
  const BwdLayout lay = bwd_layout(desc);
  if (!workspace || workspace_bytes < lay.total) return SSM_ERR_WORKSPACE;

  const void* in_ptrs[] = {x, delta, A, B, C, D, z, delta_bias, h0, dy, dhfin};
  const size_t in_bytes[] = {x_bytes, dl_bytes, a_bytes, (size_t)Bext * es, (size_t)Cext * es,
                             D ? (size_t)d.dim * 4 : 0, z ? z_bytes : 0,
                             delta_bias ? (size_t)drows * 4 : 0, h0 ? state_bytes : 0, y_bytes,
                             dhfin ? state_bytes : 0};
  constexpr int kIn = 11;
  const void* out_ptrs[] = {dx, ddelta, dz, dA, dB, dC, dD, ddelta_bias, dh0, workspace};
  const size_t out_bytes[] = {x_bytes, dl_bytes, dz ? z_bytes : 0, a_bytes, (size_t)Bext * 4,
                              (size_t)Cext * 4, dD ? (size_t)d.dim * 4 : 0,
                              ddelta_bias ? (size_t)drows * 4 : 0, dh0 ? state_bytes : 0,
                              lay.total};
  constexpr int kOut = 10;
  for (int i = 0; i < kOut; ++i) {
    for (int j = 0; j < kIn; ++j)
      if (overlaps(out_ptrs[i], out_bytes[i], in_ptrs[j], in_bytes[j])) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < kOut; ++j)
      if (overlaps(out_ptrs[i], out_bytes[i], out_ptrs[j], out_bytes[j])) return SSM_ERR_ALIAS;
  }

  ssm::BwdParams q;
  memset(&q, 0, sizeof(q));
  ssm::ScanParams& p = q.f;
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.delta_bias = delta_bias;
  p.h0 = h0;
  p.batch = d.batch; p.dim = d.dim; p.L = d.seqlen; p.N = d.dstate; p.ngroups = d.ngroups;
  p.headdim = d.headdim;
  p.x_sb = d.x_stride_batch; p.x_sd = d.x_stride_dim;
  p.dl_sb = d.delta_stride_batch; p.dl_sd = d.delta_stride_dim;
  p.B_sb = d.B_stride_batch; p.B_sg = d.B_stride_group; p.B_sn = d.B_stride_state;
  p.C_sb = d.C_stride_batch; p.C_sg = d.C_stride_group; p.C_sn = d.C_stride_state;
  p.z_sb = d.z_stride_batch; p.z_sd = d.z_stride_dim;
  p.y_sb = d.y_stride_batch; p.y_sd = d.y_stride_dim;
  p.groups_per_batch = (d.dim + ssm::kChannelsPerGroup - 1) / ssm::kChannelsPerGroup;
  p.seg_len = d.seqlen;
  p.nseg = 1;
  p.softplus = delta_softplus ? 1 : 0;
  p.zoh = disc == SSM_DISC_ZOH ? 1 : 0;
  p.ntiles = (d.seqlen + ssm::kCkptStep - 1) / ssm::kCkptStep;
  char* ws = static_cast<char*>(workspace);
  p.ckpt = reinterpret_cast<float*>(ws + lay.ckpt);
  // 16-byte rows for x, delta, dy, z (the checkpoint pass and the backward prologue)
  const int64_t vec = 16 / (int64_t)es;
  bool vec_ok = true;
  const void* vptrs[] = {x, delta, z, dy};
  for (const void* v : vptrs)
    if (v && !aligned(v, 16)) vec_ok = false;
  const int64_t vstrides[] = {d.x_stride_batch, d.x_stride_dim, d.delta_stride_batch,
                              d.delta_stride_dim, z ? d.z_stride_batch : 0, z ? d.z_stride_dim : 0,
                              d.y_stride_batch, d.y_stride_dim};
  for (int64_t st : vstrides)
    if (st % vec) vec_ok = false;
  p.vec_io = vec_ok ? 1 : 0;
  bool bc_vec = aligned(B, 16) && aligned(C, 16);
  const int64_t bstrides[] = {d.B_stride_batch, d.B_stride_group, d.B_stride_state,
                              d.C_stride_batch, d.C_stride_group, d.C_stride_state};
  for (int64_t st : bstrides)
    if (st % vec) bc_vec = false;
  p.bc_vec = bc_vec ? 1 : 0;

  q.dy = dy; q.dx = dx; q.ddelta = ddelta; q.dz = dz;
  // 16-byte stores of dx, ddelta, dz: their strides are those of x, delta, z, which vec_io
  // makes multiples of 16 bytes; the bases must be aligned too
  q.vec_out = (p.vec_io && aligned(dx, 16) && aligned(ddelta, 16) && (!dz || aligned(dz, 16)))
                  ? 1 : 0;
  q.dA = dA; q.dB = dB; q.dC = dC; q.dD = dD; q.dbias = ddelta_bias; q.dh0 = dh0;
  q.dhfin = dhfin;
  q.head = head ? 1 : 0;
  q.head_ns = ssm::bwd_wide_states_per_lane(d.dstate);
  q.span = lay.span;
  q.dB_part = reinterpret_cast<float*>(ws + lay.dB);
  q.dC_part = reinterpret_cast<float*>(ws + lay.dC);
  q.dA_part = reinterpret_cast<float*>(ws + lay.dA);
  q.dD_part = reinterpret_cast<float*>(ws + lay.dD);
  q.dbias_part = reinterpret_cast<float*>(ws + lay.dbias);
  q.ddl_part = reinterpret_cast<float*>(ws + lay.ddl);
  q.dbias_hpart = reinterpret_cast<float*>(ws + lay.dbh);
  q.part_vec = (aligned(q.dB_part, 16) && aligned(q.dC_part, 16) && d.seqlen % 4 == 0) ? 1 : 0;
  const hipError_t e = ssm::launch_bwd(q, d.io_dtype == SSM_DTYPE_BF16, hs);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_selective_scan_bwd(const ssm_scan_desc* desc, const void* x, const void* delta,
                           const float* A, const void* B, const void* C, const float* D,
                           const void* z, const float* delta_bias, int32_t delta_softplus,
                           const float* h0, const void* dy, void* dx, void* ddelta, float* dA,
                           float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                           float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  return ssm_selective_scan_bwd_ext(desc, x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0,
                                    dy, dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, nullptr,
                                    workspace, workspace_bytes, stream);
}

}  // extern "C"
