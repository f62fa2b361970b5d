/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective state-space (S6) forward scan.
 *
 * The operation (per channel d of batch b, state n, time t; all arithmetic fp32):
 *   delta_t = softplus(delta_raw_t + delta_bias)      (or delta_raw_t + delta_bias when the
 *                                                      softplus flag is 0)
 *       -- the step size is an activation of a parameter plus an input-dependent projection
 *          (page "【論文要約】Mamba: Linear-Time Sequence Modeling with Selective State
 *          Spaces【自分用メモ】", Algorithm 2 as summarised there; page "NL-345, Mamba: ...",
 *          §1 "Selection Mechanism").
 *   dA_tn   = exp(delta_t * A_n),  dB_tn = delta_t * B_tn
 *       -- the discretisation step (page "NL-345", §2 "Discretization"; A_bar as in the memo
 *          page's "数式解説" item 3; B_bar = delta * B is the simple rule the pages allow).
 *   h_tn    = dA_tn * h_(t-1)n + dB_tn * x_t,          h_(-1) = 0
 *       -- the linear recurrence, eq. (2) (page "NL-345", §2 "Computation"), one diagonal SSM per
 *          channel (same page, §2 "Structure and Dimensions").
 *   y_t     = (sum_n C_tn h_tn + D * x_t) * silu(z_t)  (the gate only when z is given)
 *       -- readout, skip term and the SiLU gate of the Mamba block (memo page, "Mambaアーキテク
 *          チャ").
 * The state h is never written to memory (memo page, "ハードウェアを考慮した効率的なアルゴリズム").
 *
 * Layouts. Every tensor is indexed with element strides given in the descriptor; the time
 * (L) stride is always 1:
 *   x, z, y     (batch, dim, L)                        io dtype
 *   delta       (batch, dim, L)   A_DIAG mode          io dtype
 *               (batch, nheads, L) A_HEAD mode (nheads = dim / headdim)
 *   A           (dim, dstate) fp32 contiguous, A_DIAG mode; (nheads,) fp32 in A_HEAD mode
 *   B, C        (batch, ngroups, dstate, L)            io dtype; channel d reads group
 *                                                       d / (dim / ngroups)
 *   D           (dim,) fp32, nullable (treated as 0)
 *   delta_bias  (dim,) fp32 in A_DIAG mode, (nheads,) in A_HEAD mode; nullable (treated as 0)
 *   z           nullable: no gate
 * Channel d belongs to head d / headdim (A_HEAD mode).
 *
 * Ownership and execution: the caller owns every buffer (device memory) and the stream. The
 * library allocates nothing and keeps no mutable global state; calls are thread-safe. Work is
 * enqueued asynchronously on `stream` (a hipStream_t, NULL = the default stream). Device faults
 * surface at the caller's next synchronisation.
 *
 * Errors: every entry point returns SSM_OK (0) or a negative ssm_status. Argument checks run on
 * the host before anything is enqueued; on an error nothing is launched and no buffer is touched.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_ABI_VERSION 6

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL_ARG = -1,       /* a required pointer (desc, x, delta, A, B, C, y) is NULL */
  SSM_ERR_BAD_SHAPE = -2,      /* a size < 0, dim/dstate/ngroups/headdim < 1, dim % ngroups,
                                  dim % headdim, dstate > SSM_MAX_DSTATE (128), or sizes that overflow */
  SSM_ERR_BAD_DTYPE = -3,      /* io_dtype, a_mode, discretization or algorithm not one of the
                                  enums below */
  SSM_ERR_BAD_STRIDE = -4,     /* a negative stride, or strides that make the rows of an output
                                  overlap (the rows of a tensor are disjoint when, taken by
                                  increasing stride, each dimension of size > 1 steps past the
                                  whole extent of the dimensions below it) */
  SSM_ERR_MISALIGNED = -5,     /* a pointer not aligned to its element size */
  SSM_ERR_ALIAS = -6,          /* an output (y, h_final, workspace) overlaps an input or another
                                  output */
  SSM_ERR_WORKSPACE = -7,      /* workspace NULL or smaller than the size query returns */
  SSM_ERR_HIP = -8,            /* the HIP runtime reported an error while enqueueing */
  SSM_ERR_UNSUPPORTED = -9,    /* valid arguments outside what this build implements */
  SSM_ERR_SCRATCH_LIMIT = -10  /* ssm_selective_scan_fwd_noalloc: the problem needs more scratch
                                  than the library's fixed array holds */
} ssm_status;

typedef enum { SSM_DTYPE_F32 = 0, SSM_DTYPE_BF16 = 1 } ssm_dtype;

typedef enum {
  SSM_A_DIAG = 0,   /* A is (dim, dstate): a diagonal A per channel, delta per channel */
  SSM_A_HEAD = 1,   /* A is one scalar per head; delta and delta_bias per head */
  SSM_A_COMPLEX = 2 /* A is (dim, dstate) complex, stored as (dim, dstate, 2) fp32 pairs
                       (real, imaginary); B and C are complex: each (batch, group) holds 2*dstate
                       rows, the real parts at state rows 0..dstate-1 and the imaginary parts at
                       rows dstate..2*dstate-1 (B_stride_state / C_stride_state between rows);
                       the state is complex and y_t = Re(sum_n C_tn h_tn) + D x_t (times the
                       gate). delta, delta_bias as in SSM_A_DIAG; headdim must be 1. The memo
                       page's Figure 10 caption compares SSM parameterisations and stresses
                       complex-valued parameters; the pages give no formula, so the recurrence
                       above is taken over complex numbers. Forward scan only (see
                       ssm_selective_scan_fwd_ext); dstate <= SSM_MAX_COMPLEX_DSTATE. */
} ssm_a_mode;

#define SSM_MAX_COMPLEX_DSTATE 32

#define SSM_MAX_DSTATE 128

typedef struct ssm_scan_desc {
  int64_t batch;    /* >= 0 */
  int64_t dim;      /* channels (d_inner), >= 1 */
  int64_t seqlen;   /* L, >= 0 */
  int64_t dstate;   /* N, 1..SSM_MAX_DSTATE (128) */
  int64_t ngroups;  /* B/C groups, >= 1, divides dim */
  int64_t headdim;  /* channels per head, >= 1, divides dim; 1 in A_DIAG mode */
  int32_t io_dtype; /* ssm_dtype of x, delta, B, C, z and y */
  int32_t a_mode;   /* ssm_a_mode */
  /* element strides (the L stride is 1) */
  int64_t x_stride_batch, x_stride_dim;
  int64_t delta_stride_batch, delta_stride_dim; /* dim index: channel (DIAG) or head (HEAD) */
  int64_t B_stride_batch, B_stride_group, B_stride_state;
  int64_t C_stride_batch, C_stride_group, C_stride_state;
  int64_t z_stride_batch, z_stride_dim;
  int64_t y_stride_batch, y_stride_dim;
} ssm_scan_desc;

/* Fills `desc` with the contiguous layout of the given sizes (strides as listed above, L
 * innermost; with SSM_A_COMPLEX, B and C have 2 * dstate rows per group). Returns SSM_ERR_NULL_ARG for a NULL desc, else SSM_OK; sizes are checked by the
 * calls that use the descriptor. */
int ssm_scan_desc_init_contiguous(ssm_scan_desc* desc, int64_t batch, int64_t dim, int64_t seqlen,
                                  int64_t dstate, int64_t ngroups, int64_t headdim,
                                  int32_t io_dtype, int32_t a_mode);

/* Bytes of device workspace that ssm_selective_scan_fwd needs for `desc` (0 when the sequence
 * is processed in one segment). The value depends only on the descriptor. */
int ssm_selective_scan_workspace_size(const ssm_scan_desc* desc, size_t* bytes);

/* The selective-scan forward pass described at the top of this header.
 *   x, delta, B, C, z, y : device pointers of the io dtype (z may be NULL)
 *   A, D, delta_bias     : device pointers, fp32 (D and delta_bias may be NULL)
 *   delta_softplus       : nonzero applies softplus to delta_raw + delta_bias
 *   workspace            : device scratch of at least the queried size, 4-byte aligned (may be
 *                          NULL when the query returns 0); its contents on entry do not matter
 *                          and it must not overlap any other argument
 *   stream               : hipStream_t to enqueue on
 * y must not overlap any input. */
int ssm_selective_scan_fwd(const ssm_scan_desc* desc, const void* x, const void* delta,
                           const float* A, const void* B, const void* C, const float* D,
                           const void* z, const float* delta_bias, int32_t delta_softplus,
                           void* y, void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* ssm_status_string(int status);

/* Discretisation of B (the pages' f_B).
 *   SSM_DISC_DELTA_B: B_bar = delta * B (the default).
 *   SSM_DISC_ZOH:     B_bar = (exp(delta A) - 1) / A * B, the zero-order hold; it tends to
 *                     delta * B as delta A -> 0 and equals it where A == 0. (Page "NL-345",
 *                     §2 "Discretization", eq. (4); memo page, "数式解説".) */
typedef enum { SSM_DISC_DELTA_B = 0, SSM_DISC_ZOH = 1 } ssm_discretization;

/* How the forward pass evaluates the scan. Both compute the same recurrence.
 *   SSM_ALGO_AUTO:      the chunked form where it applies (below), else the recurrent one.
 *   SSM_ALGO_RECURRENT: the recurrence step by step, fp32 arithmetic throughout.
 *   SSM_ALGO_CHUNKED:   the block decomposition of the semiseparable matrix (review page of
 *                       "Transformers are SSMs", proposed method: the SSD algorithm): per chunk
 *                       of 64 steps a masked, decay-weighted quadratic product inside the chunk
 *                       and a state of dstate x 64 channels passed between chunks, evaluated as
 *                       bf16 matrix products with fp32 accumulation and an fp32 state. It applies
 *                       to io_dtype BF16, a_mode HEAD, headdim a multiple of 64, dstate 64 or
 *                       128, dim / ngroups a multiple of 64, 16-byte aligned x, delta, z, y, B, C,
 *                       h0 and h_final with strides that are multiples of 8 elements. Requested
 *                       outside that it returns SSM_ERR_UNSUPPORTED. It needs no workspace. */
typedef enum { SSM_ALGO_AUTO = 0, SSM_ALGO_RECURRENT = 1, SSM_ALGO_CHUNKED = 2 } ssm_algorithm;

/* Options of ssm_selective_scan_fwd_ext. A zero-filled struct gives ssm_selective_scan_fwd.
 * The state carried between calls lets a long sequence be scanned in pieces (the recurrence is
 * the same across a call boundary: page "NL-345", §2 "Computation", recurrent mode). */
typedef struct ssm_scan_ext {
  int32_t discretization; /* ssm_discretization */
  int32_t algorithm;      /* ssm_algorithm */
  const float* h0;        /* nullable: initial state (batch, dim, dstate) fp32, contiguous, read
                             before the first step; NULL starts from zeros */
  float* h_final;         /* nullable: receives the state after the last step, (batch, dim,
                             dstate) fp32 contiguous; must not overlap h0, y or any input (use
                             two buffers to carry the state across calls) */
} ssm_scan_ext;

/* ssm_selective_scan_fwd with the options above (`ext` may be NULL). With seqlen == 0, y is not
 * touched and h_final receives h0 (or zeros). The workspace size does not depend on `ext`.
 * a_mode SSM_A_COMPLEX takes the delta * B rule, no h0 or h_final and the recurrent algorithm
 * (AUTO or RECURRENT), with dstate <= SSM_MAX_COMPLEX_DSTATE; it needs no workspace. Any other
 * option with it returns SSM_ERR_UNSUPPORTED. */
int ssm_selective_scan_fwd_ext(const ssm_scan_desc* desc, const void* x, const void* delta,
                               const float* A, const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, int32_t delta_softplus,
                               void* y, const ssm_scan_ext* ext, void* workspace,
                               size_t workspace_bytes, void* stream);

/* One recurrent step per sequence, for decoding one token at a time (a_mode DIAG or HEAD; COMPLEX
 * returns SSM_ERR_UNSUPPORTED): the state carries the
 * whole history, so each step costs the same whatever the position (page "NL-345", §1
 * "Selection Mechanism" and §2 "Computation": the recurrent mode of a selective SSM).
 *   `desc` describes a scan with seqlen == 1 (SSM_ERR_BAD_SHAPE otherwise): x, delta, z, y are
 *   (batch, dim | nheads, 1) and B, C (batch, ngroups, dstate, 1), with the usual strides.
 *   state (batch, dim, dstate) fp32 contiguous is read and overwritten in place:
 *     state <- exp(delta A) state + delta B x,   y = C.state + D x   (times silu(z))
 *   with delta = softplus(delta_raw + delta_bias) as in the scan; B_bar is delta * B.
 * state and y must not overlap any input or each other. Asynchronous on `stream`; no workspace. */
int ssm_selective_state_update(const ssm_scan_desc* desc, float* state, const void* x,
                               const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias,
                               int32_t delta_softplus, void* y, void* stream);

/* Bytes of device workspace that ssm_selective_scan_bwd needs for `desc` (0 when batch or
 * seqlen is 0). The value depends only on the descriptor. */
int ssm_selective_scan_bwd_workspace_size(const ssm_scan_desc* desc, size_t* bytes);

/* Gradients of ssm_selective_scan_fwd with respect to every input, given dy, the gradient of its
 * output y: the backward half of training the layer (page "NL-345", §1 "Hardware-aware
 * Algorithm": the states are recomputed from sparse checkpoints, not stored).
 *   inputs   : the forward call's desc, x, delta, A, B, C, D, z, delta_bias, delta_softplus and
 *              h0 (nullable initial state, (batch, dim, dstate) fp32 contiguous)
 *   dy       : io dtype with the strides of y
 *   dx       : io dtype, strides of x;  ddelta: io dtype, strides of delta (gradient of the raw
 *              delta, before bias and softplus; (batch, nheads, L) in A_HEAD mode);  dz: io
 *              dtype, strides of z (required when z is given, ignored otherwise)
 *   dB, dC   : fp32 with the element strides of B and C (summed over the channels of a group)
 *   dA       : fp32 shaped like A ((dim, dstate), or (nheads,) in A_HEAD mode);  dD (dim,) and
 *              ddelta_bias (shaped like delta_bias), fp32, nullable (not computed); summed over
 *              the batch (and over each head's channels in A_HEAD mode)
 *   dh0      : nullable, (batch, dim, dstate) fp32: the gradient of the initial state
 *   workspace: at least ssm_selective_scan_bwd_workspace_size bytes, 4-byte aligned
 * The a_modes DIAG and HEAD, every io dtype and dstate up to 128 are supported (COMPLEX returns
 * SSM_ERR_UNSUPPORTED). Outputs must not overlap any input
 * or each other. Because dx, ddelta, dz, dB and dC are written with the strides of x, delta, z,
 * B and C, those strides must give disjoint rows (as y's must in the forward call; a stride-0
 * broadcast of B, say, returns SSM_ERR_BAD_STRIDE). Results are deterministic (fixed-order
 * reductions). This is the delta * B rule with no final-state gradient; see
 * ssm_selective_scan_bwd_ext for the others. */
int ssm_selective_scan_bwd(const ssm_scan_desc* desc, const void* x, const void* delta,
                           const float* A, const void* B, const void* C, const float* D,
                           const void* z, const float* delta_bias, int32_t delta_softplus,
                           const float* h0, const void* dy, void* dx, void* ddelta, float* dA,
                           float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                           float* dh0, void* workspace, size_t workspace_bytes, void* stream);

/* Options of ssm_selective_scan_bwd_ext. A zero-filled struct gives ssm_selective_scan_bwd. */
typedef struct ssm_bwd_ext {
  int32_t discretization; /* the ssm_discretization of the forward call (the zero-order hold
                             differentiates B_bar = (exp(delta A) - 1) / A B) */
  int32_t reserved;       /* 0 */
  const float* dh_final;  /* nullable: gradient of the forward call's final state (batch, dim,
                             dstate) fp32 contiguous, for a sequence scanned in pieces; NULL is
                             a zero gradient */
} ssm_bwd_ext;

/* ssm_selective_scan_bwd with the options above (`ext` may be NULL): the gradients of
 * ssm_selective_scan_fwd_ext with the given discretisation, including the gradient that flows
 * in through its final state. Arguments, layouts and errors as ssm_selective_scan_bwd. With
 * batch or seqlen 0 the parameter gradients are zero and dh0 receives dh_final (or zeros). */
int ssm_selective_scan_bwd_ext(const ssm_scan_desc* desc, const void* x, const void* delta,
                               const float* A, const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, int32_t delta_softplus,
                               const float* h0, const void* dy, void* dx, void* ddelta,
                               float* dA, float* dB, float* dC, float* dD, void* dz,
                               float* ddelta_bias, float* dh0, const ssm_bwd_ext* ext,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Size of the fixed device array that ssm_selective_scan_fwd_noalloc uses as its workspace:
 * 8 MiB, held on every GPU the library runs on until the process ends. The per-segment
 * summaries of every segment plan with dstate <= 32 fit it (2.2 MB for the million-token scan).
 * A split sequence's workspace also holds states that let the pass correcting its later
 * segments stop early (64 MiB for the million-token scan); where those do not fit, the array
 * holds the summaries only and that pass runs every later segment to its end: the results are
 * the same, only slower. */
#define SSM_NOALLOC_SCRATCH_BYTES (8 << 20)

/* ssm_selective_scan_fwd_ext for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same computation
 * and results, with the workspace taken from a fixed device array of SSM_NOALLOC_SCRATCH_BYTES
 * owned by the library instead of a caller buffer. It allocates nothing and calls no
 * allocating routine. The caller still passes every input and output.
 *   Arguments, layouts and errors: those of ssm_selective_scan_fwd_ext (`ext` may be NULL).
 *   Returns SSM_ERR_SCRATCH_LIMIT, before touching the GPU, when even the summaries alone (see
 *   SSM_NOALLOC_SCRATCH_BYTES) exceed SSM_NOALLOC_SCRATCH_BYTES, and SSM_ERR_HIP
 *   when the array's device address cannot be found. The first call on a device looks that
 *   address up (with the stream's device current) and keeps it.
 *   Every call on a GPU shares that GPU's array and leaves its contents behind; nothing in it
 *   needs to start at zero. Calls on one stream are ordered; calls whose work overlaps on one
 *   GPU (two streams, or two host threads without ordering) race on the array. */
int ssm_selective_scan_fwd_noalloc(const ssm_scan_desc* desc, const void* x, const void* delta,
                                   const float* A, const void* B, const void* C, const float* D,
                                   const void* z, const float* delta_bias, int32_t delta_softplus,
                                   void* y, const ssm_scan_ext* ext, void* stream);

/* SSM_SCAN_ABI_VERSION of the built library. */
int ssm_abi_version(void);

/* Diagnostic of a hardware assumption, no part of the scan: launches `nworkgroups` workgroups of
 * eight wavefronts, the shape of the forward kernel with independent wavefronts, and writes to
 * out[8 g + w] (device memory of 8 * nworkgroups int32, caller-owned) the SIMD (0..3 of its
 * compute unit) that wavefront w of workgroup g ran on. That kernel paces wavefronts w and w ^ 4
 * of a workgroup against each other on the assumption that they share a SIMD; a test checks it.
 * Returns SSM_ERR_NULL_ARG for a null `out` and SSM_ERR_BAD_SHAPE for a negative count (nothing
 * is launched), else SSM_OK or SSM_ERR_HIP (launch failure). Runs asynchronously on `stream`. */
int ssm_wave_simd_ids(int32_t* out, int32_t nworkgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
