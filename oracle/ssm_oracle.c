/*
 * CPU ORACLE for the selective state-space (S6) forward scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load this library. It
 * shares no code with the HIP path. It is deliberately plain: fp64 throughout, one channel at a
 * time, time steps in order, states in order, no blocking, fusion or reordering.
 *
 * What it computes, and where each step is defined:
 *   - Selection (page "【論文要約】Mamba: Linear-Time Sequence Modeling with Selective State
 *     Spaces【自分用メモ】", Algorithm 2 as summarised there; page "NL-345, Mamba: ...", §1
 *     Selection Mechanism): the step size is delta = tau(bias + Delta_raw), tau = softplus;
 *     A is a fixed parameter, B and C arrive already input-dependent.
 *   - Discretisation (page "NL-345, Mamba: ...", §2 State Space Models, "Discretization": a
 *     rule (f_A, f_B); the memo page, "数式解説" item 3, ZOH): A_bar = exp(delta * A) and
 *     either B_bar = delta * B (default) or the zero-order hold
 *     B_bar = (delta A)^-1 (exp(delta A) - 1) delta B = expm1(delta A) / A * B.
 *   - Recurrence (page "NL-345", §2 "Computation", eq. (2); the memo page, "数式解説" item 2):
 *     h_t = A_bar_t h_{t-1} + B_bar_t x_t, y_t = C_t h_t.
 *   - Diagonal structure, one independent SSM per channel (page "NL-345", §2 "Structure and
 *     Dimensions"): A, B, C are N numbers each; the state is N per channel.
 *   - Skip and gate: y_t <- (C_t . h_t + D x_t) * silu(z_t), silu(z) = z / (1 + exp(-z)) (the
 *     memo page, "Mambaアーキテクチャ": SiLU activation in the block).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   initial state h_{-1} = 0 unless h0 is given; the bias is added before softplus and also when
 *   softplus is off; softplus(v) = log(1 + e^v) evaluated as max(v,0) + log1p(exp(-|v|)); the
 *   gate multiplies the skip term too.
 *
 * Layouts (all fp64, L contiguous):
 *   x, z, y   [batch][dim][L]
 *   delta     [batch][dim][L] (per-channel mode) or [batch][nheads][L] (head mode)
 *   A         [dim][N] (per-channel mode) or [nheads] (head mode: one scalar per head)
 *   B, C      [batch][ngroups][N][L]
 *   D         [dim] or NULL (= 0); delta_bias [dim] / [nheads] or NULL (= 0)
 *   h0, hT    [batch][dim][N] or NULL
 * Channel d belongs to head d / headdim and to group d / (dim / ngroups).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t batch, dim, L, N, ngroups, headdim;
  int head_mode, delta_softplus, zoh;
  const double *x, *delta, *A, *B, *C, *D, *z, *delta_bias, *h0;
  double *y, *hT;
} oracle_problem;

static double softplus(double v) {
  /* log(1 + e^v) without overflow or cancellation */
  return (v > 0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One channel (b, d): the sequential recurrence over t = 0..L-1. */
static void scan_channel(const oracle_problem* p, int64_t b, int64_t d, double* h) {
  const int64_t L = p->L, N = p->N;
  const int64_t nheads = p->dim / p->headdim;
  const int64_t head = d / p->headdim;
  const int64_t group = d / (p->dim / p->ngroups);
  const int64_t dch = p->head_mode ? head : d;  /* row of delta / delta_bias */
  const int64_t drows = p->head_mode ? nheads : p->dim;
  const double* xr = p->x + (b * p->dim + d) * L;
  const double* dr = p->delta + (b * drows + dch) * L;
  const double* Bg = p->B + (b * p->ngroups + group) * N * L;
  const double* Cg = p->C + (b * p->ngroups + group) * N * L;
  const double* zr = p->z ? p->z + (b * p->dim + d) * L : NULL;
  double* yr = p->y + (b * p->dim + d) * L;
  const double bias = p->delta_bias ? p->delta_bias[dch] : 0.0;
  const double Dd = p->D ? p->D[d] : 0.0;

  for (int64_t n = 0; n < N; ++n) h[n] = p->h0 ? p->h0[(b * p->dim + d) * N + n] : 0.0;

  for (int64_t t = 0; t < L; ++t) {
    const double v = dr[t] + bias;
    const double delta = p->delta_softplus ? softplus(v) : v;
    const double xt = xr[t];
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = p->head_mode ? p->A[head] : p->A[d * N + n];
      const double Bt = Bg[n * L + t], Ct = Cg[n * L + t];
      /* discretise */
      const double Abar = exp(delta * a);
      double Bbar;
      if (p->zoh) Bbar = (a != 0.0) ? expm1(delta * a) / a * Bt : delta * Bt;
      else Bbar = delta * Bt;
      /* recur and read out */
      h[n] = Abar * h[n] + Bbar * xt;
      acc += Ct * h[n];
    }
    double yt = acc + Dd * xt;
    if (zr) yt *= silu(zr[t]);
    yr[t] = yt;
  }
  if (p->hT)
    for (int64_t n = 0; n < N; ++n) p->hT[(b * p->dim + d) * N + n] = h[n];
}

typedef struct { const oracle_problem* p; int64_t lo, hi; int rc; } oracle_part;

static void* oracle_worker(void* arg) {
  oracle_part* w = (oracle_part*)arg;
  double hbuf[1024];
  for (int64_t c = w->lo; c < w->hi; ++c) scan_channel(w->p, c / w->p->dim, c % w->p->dim, hbuf);
  return NULL;
}

/*
 * Runs the scan for every (b, d) channel, channels split statically over nthreads POSIX threads.
 * Returns 0, or -1 on inconsistent sizes (N > 1024, dim not divisible by headdim/ngroups, ...).
 */
int ssm_oracle_scan(int64_t batch, int64_t dim, int64_t L, int64_t N, int64_t ngroups,
                    int64_t headdim, int head_mode, int delta_softplus, int zoh,
                    const double* x, const double* delta, const double* A, const double* B,
                    const double* C, const double* D, const double* z, const double* delta_bias,
                    const double* h0, double* y, double* hT, int nthreads) {
  if (batch < 0 || dim < 1 || L < 0 || N < 1 || N > 1024 || ngroups < 1 || headdim < 1) return -1;
  if (dim % ngroups || dim % headdim) return -1;
  if (!x || !delta || !A || !B || !C || !y) return -1;
  oracle_problem p = {batch, dim, L, N, ngroups, headdim, head_mode, delta_softplus, zoh,
                      x, delta, A, B, C, D, z, delta_bias, h0, y, hT};
  const int64_t channels = batch * dim;
  if (channels == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > channels) nthreads = (int)channels;
  pthread_t th[256];
  oracle_part parts[256];
  int64_t per = (channels + nthreads - 1) / nthreads;
  int started[256] = {0};
  for (int t = 0; t < nthreads; ++t) {
    parts[t].p = &p;
    parts[t].lo = per * t;
    parts[t].hi = per * (t + 1) < channels ? per * (t + 1) : channels;
    parts[t].rc = 0;
    if (parts[t].lo >= parts[t].hi) continue;
    if (nthreads == 1 || pthread_create(&th[t], NULL, oracle_worker, &parts[t]) != 0)
      oracle_worker(&parts[t]);
    else
      started[t] = 1;
  }
  for (int t = 0; t < nthreads; ++t) if (started[t]) pthread_join(th[t], NULL);
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Gradients of the scan above (reverse-mode differentiation of the same loop, written out; the
 * pages train the model end to end, so the scan's backward pass is the other half of its hot
 * path: page "NL-345", §1 "Hardware-aware Algorithm", which recomputes states for it).
 *
 * Given gy_out = dL/dy for the gated output y, the chain rule through one step of the loop
 * (h_t = Abar_t h_{t-1} + Bbar_t x_t, Abar = exp(delta a), y_t = (C_t . h_t + D x_t) g(z_t)):
 *   gy      = gy_out * silu(z)                      (the gradient of the ungated readout)
 *   dz      = gy_out * (C . h + D x) * silu'(z),     silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
 *   gh_t   += gy C_t                                 (gh_t accumulates dL/dh_t from step t and,
 *                                                     through gh_t = Abar_{t+1} gh_{t+1}, later)
 *   dC_t   += gy h_t,  dD += gy x_t,  dx_t = gy D + sum_n gh_t Bbar_t
 *   ddelta  = sum_n gh_t (a Abar_t h_{t-1} + x_t dBbar/ddelta),   dBbar/ddelta = B (delta*B rule)
 *                                                                 or Abar B (zero-order hold)
 *   da     += gh_t (delta Abar_t h_{t-1} + x_t dBbar/da),   dBbar/da = 0, or
 *                                          B (delta a Abar - expm1(delta a)) / a^2 (ZOH)
 *   dB_t   += gh_t x_t Bbar_t / B_t,  dh_{t-1} = Abar_t gh_t,
 *   ddelta_raw = ddelta * sigmoid(delta_raw + bias) under softplus (its derivative), else
 *   ddelta; dbias += ddelta_raw.
 * The states h_t are recomputed by a forward pass and kept for the whole sequence.
 * Layouts as for the forward; dB, dC are [batch][ngroups][N][L], dA is [dim][N] (or [nheads]),
 * dD [dim], ddelta_bias [dim] (or [nheads]), dh0 [batch][dim][N]. Any of dD, dz, ddelta_bias,
 * dh0 may be NULL (not wanted). dh_final [batch][dim][N], the gradient of the state after the
 * last step (nonzero when the sequence continues in a later call), may be NULL (zero); dh0 is
 * the gradient of the initial state. Gradients of values shared by several channels (B, C, and
 * delta, A, bias in head mode, A, D, bias across the batch) are sums over those channels; the
 * sums over the batch run in batch order, so results do not depend on the thread count.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  const oracle_problem* p;
  const double* dy;
  const double* dh_final;  /* gradient of the state after the last step, or NULL (zero) */
  double *dx, *ddelta, *dB, *dC, *dz, *dh0;
  double *dA_b, *dD_b, *dbias_b;  /* per batch entry: [batch][dim*N or nheads], [batch][dim], ... */
} bwd_problem;

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

static void bwd_channel(const bwd_problem* q, int64_t b, int64_t d, double* hist, double* gh) {
  const oracle_problem* p = q->p;
  const int64_t L = p->L, N = p->N;
  const int64_t nheads = p->dim / p->headdim;
  const int64_t head = d / p->headdim;
  const int64_t group = d / (p->dim / p->ngroups);
  const int64_t dch = p->head_mode ? head : d;
  const int64_t drows = p->head_mode ? nheads : p->dim;
  const double* xr = p->x + (b * p->dim + d) * L;
  const double* dr = p->delta + (b * drows + dch) * L;
  const double* Bg = p->B + (b * p->ngroups + group) * N * L;
  const double* Cg = p->C + (b * p->ngroups + group) * N * L;
  const double* zr = p->z ? p->z + (b * p->dim + d) * L : NULL;
  const double* gyr = q->dy + (b * p->dim + d) * L;
  double* dBg = q->dB + (b * p->ngroups + group) * N * L;
  double* dCg = q->dC + (b * p->ngroups + group) * N * L;
  double* dxr = q->dx + (b * p->dim + d) * L;
  double* ddr = q->ddelta + (b * drows + dch) * L;
  double* dzr = q->dz && zr ? q->dz + (b * p->dim + d) * L : NULL;
  const double bias = p->delta_bias ? p->delta_bias[dch] : 0.0;
  const double Dd = p->D ? p->D[d] : 0.0;

  /* forward pass, keeping h_{t} in hist[(t + 1) * N + n] (hist[n] is the initial state) */
  for (int64_t n = 0; n < N; ++n) hist[n] = p->h0 ? p->h0[(b * p->dim + d) * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double v = dr[t] + bias;
    const double delta = p->delta_softplus ? softplus(v) : v;
    for (int64_t n = 0; n < N; ++n) {
      const double a = p->head_mode ? p->A[head] : p->A[d * N + n];
      const double Bt = Bg[n * L + t];
      const double Bbar = p->zoh ? ((a != 0.0) ? expm1(delta * a) / a * Bt : delta * Bt) : delta * Bt;
      hist[(t + 1) * N + n] = exp(delta * a) * hist[t * N + n] + Bbar * xr[t];
    }
  }

  /* reverse pass: gh starts as dL/dh_{L-1}, the gradient of the final state (the recurrence
   * goes on across a call boundary, so a later piece of the sequence hands it back) */
  for (int64_t n = 0; n < N; ++n)
    gh[n] = q->dh_final ? q->dh_final[(b * p->dim + d) * N + n] : 0.0;
  double dD = 0.0, dbias = 0.0;
  for (int64_t t = L - 1; t >= 0; --t) {
    const double v = dr[t] + bias;
    const double delta = p->delta_softplus ? softplus(v) : v;
    const double xt = xr[t];
    const double* ht = hist + (t + 1) * N;
    const double* hp = hist + t * N;
    double gy = gyr[t];
    if (zr) {
      double pre = Dd * xt;
      for (int64_t n = 0; n < N; ++n) pre += Cg[n * L + t] * ht[n];
      const double s = sigmoid(zr[t]);
      if (dzr) dzr[t] = gyr[t] * pre * s * (1.0 + zr[t] * (1.0 - s));
      gy = gyr[t] * zr[t] * s;
    }
    dD += gy * xt;
    double gx = gy * Dd, gdelta = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = p->head_mode ? p->A[head] : p->A[d * N + n];
      const double Bt = Bg[n * L + t], Ct = Cg[n * L + t];
      const double Abar = exp(delta * a);
      /* Bbar = f * Bt with f = delta, or f = expm1(delta a) / a under the zero-order hold */
      double f, df_ddelta, df_da;
      if (p->zoh && a != 0.0) {
        f = expm1(delta * a) / a;
        df_ddelta = Abar;
        df_da = (delta * a * Abar - expm1(delta * a)) / (a * a);
      } else if (p->zoh) {  /* a == 0: f = delta, and d/da of expm1(delta a)/a at 0 is delta^2/2 */
        f = delta;
        df_ddelta = 1.0;
        df_da = delta * delta * 0.5;
      } else {
        f = delta;
        df_ddelta = 1.0;
        df_da = 0.0;
      }
      const double Bbar = f * Bt;
      const double dBbar_ddelta = df_ddelta * Bt, dBbar_da = df_da * Bt;
      gh[n] += gy * Ct;
      dCg[n * L + t] += gy * ht[n];
      dBg[n * L + t] += gh[n] * xt * f;
      gdelta += gh[n] * (a * Abar * hp[n] + xt * dBbar_ddelta);
      const double da = gh[n] * (delta * Abar * hp[n] + xt * dBbar_da);
      if (p->head_mode) q->dA_b[b * nheads + head] += da;
      else q->dA_b[(b * p->dim + d) * N + n] += da;
      gx += gh[n] * Bbar;
      gh[n] *= Abar;
    }
    const double gv = p->delta_softplus ? gdelta * sigmoid(v) : gdelta;
    if (p->head_mode) ddr[t] += gv;
    else ddr[t] = gv;
    dbias += gv;
    dxr[t] = gx;
  }
  q->dD_b[b * p->dim + d] = dD;
  q->dbias_b[b * drows + dch] += dbias;
  if (q->dh0)
    for (int64_t n = 0; n < N; ++n) q->dh0[(b * p->dim + d) * N + n] = gh[n];
}

typedef struct { const bwd_problem* q; int64_t lo, hi; double* hist; double* gh; } bwd_part;

static void* bwd_worker(void* arg) {
  bwd_part* w = (bwd_part*)arg;
  const oracle_problem* p = w->q->p;
  for (int64_t b = w->lo; b < w->hi; ++b)
    for (int64_t d = 0; d < p->dim; ++d) bwd_channel(w->q, b, d, w->hist, w->gh);
  return NULL;
}

/*
 * Gradients of ssm_oracle_scan for every input. Threads split the batch entries (each entry's
 * channels in order on one thread); the per-entry contributions to dA, dD and ddelta_bias are
 * then summed over the batch in order. hist is an (L + 1) * N fp64 buffer per thread.
 * Returns 0, or -1 on inconsistent sizes or a failed allocation.
 */
int ssm_oracle_scan_bwd(int64_t batch, int64_t dim, int64_t L, int64_t N, int64_t ngroups,
                        int64_t headdim, int head_mode, int delta_softplus, int zoh,
                        const double* x, const double* delta, const double* A, const double* B,
                        const double* C, const double* D, const double* z,
                        const double* delta_bias, const double* h0, const double* dy,
                        const double* dh_final, double* dx, double* ddelta, double* dA,
                        double* dB, double* dC, double* dD, double* dz, double* ddelta_bias,
                        double* dh0, int nthreads) {
  if (batch < 0 || dim < 1 || L < 0 || N < 1 || N > 1024 || ngroups < 1 || headdim < 1) return -1;
  if (dim % ngroups || dim % headdim) return -1;
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return -1;
  oracle_problem p = {batch, dim, L, N, ngroups, headdim, head_mode, delta_softplus, zoh,
                      x, delta, A, B, C, D, z, delta_bias, h0, NULL, NULL};
  const int64_t nheads = dim / headdim;
  const int64_t drows = head_mode ? nheads : dim;
  const int64_t a_count = head_mode ? nheads : dim * N;
  memset(ddelta, 0, sizeof(double) * (size_t)(batch * drows * L));
  memset(dB, 0, sizeof(double) * (size_t)(batch * ngroups * N * L));
  memset(dC, 0, sizeof(double) * (size_t)(batch * ngroups * N * L));
  double* dA_b = calloc((size_t)(batch * a_count + 1), sizeof(double));
  double* dD_b = calloc((size_t)(batch * dim + 1), sizeof(double));
  double* dbias_b = calloc((size_t)(batch * drows + 1), sizeof(double));
  if (!dA_b || !dD_b || !dbias_b) { free(dA_b); free(dD_b); free(dbias_b); return -1; }
  bwd_problem q = {&p, dy, dh_final, dx, ddelta, dB, dC, dz, dh0, dA_b, dD_b, dbias_b};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > batch) nthreads = (int)(batch > 0 ? batch : 1);
  pthread_t th[256];
  bwd_part parts[256];
  int started[256] = {0};
  int rc = 0;
  const int64_t per = batch > 0 ? (batch + nthreads - 1) / nthreads : 0;
  for (int t = 0; t < nthreads; ++t) {
    parts[t].q = &q;
    parts[t].lo = per * t;
    parts[t].hi = per * (t + 1) < batch ? per * (t + 1) : batch;
    parts[t].hist = malloc(sizeof(double) * (size_t)((L + 1) * N));
    parts[t].gh = malloc(sizeof(double) * (size_t)N);
    if (!parts[t].hist || !parts[t].gh) rc = -1;
  }
  for (int t = 0; t < nthreads && rc == 0; ++t) {
    if (parts[t].lo >= parts[t].hi) continue;
    if (nthreads == 1 || pthread_create(&th[t], NULL, bwd_worker, &parts[t]) != 0)
      bwd_worker(&parts[t]);
    else
      started[t] = 1;
  }
  for (int t = 0; t < nthreads; ++t) if (started[t]) pthread_join(th[t], NULL);
  if (rc == 0) {
    for (int64_t i = 0; i < a_count; ++i) {
      double s = 0.0;
      for (int64_t b = 0; b < batch; ++b) s += dA_b[b * a_count + i];
      dA[i] = s;
    }
    if (dD)
      for (int64_t i = 0; i < dim; ++i) {
        double s = 0.0;
        for (int64_t b = 0; b < batch; ++b) s += dD_b[b * dim + i];
        dD[i] = s;
      }
    if (ddelta_bias)
      for (int64_t i = 0; i < drows; ++i) {
        double s = 0.0;
        for (int64_t b = 0; b < batch; ++b) s += dbias_b[b * drows + i];
        ddelta_bias[i] = s;
      }
  }
  for (int t = 0; t < nthreads; ++t) { free(parts[t].hist); free(parts[t].gh); }
  free(dA_b); free(dD_b); free(dbias_b);
  return rc;
}

/* ------------------------------------------------------------------------------------------
 * Complex diagonal A. The memo page's Figure 10 caption compares SSM parameterisations on audio
 * and stresses that complex-valued parameters matter there; the pages give no formula for that
 * case. The reading taken here is the recurrence above with complex numbers:
 *   A_n complex per (channel, state); B_tn, C_tn complex (input-dependent, per group);
 *   delta, x, z real;  A_bar = exp(delta A) (complex exponential), B_bar = delta B;
 *   h_t = A_bar_t h_{t-1} + B_bar_t x_t (complex state);  y_t = Re(sum_n C_tn h_tn) + D x_t,
 *   times silu(z_t).
 * Layouts (fp64): Ar, Ai [dim][N]; Br, Bi, Cr, Ci [batch][ngroups][N][L]; the rest as above.
 * -------------------------------------------------------------------------------------------*/
#include <complex.h>

typedef struct {
  int64_t batch, dim, L, N, ngroups;
  int delta_softplus;
  const double *x, *delta, *Ar, *Ai, *Br, *Bi, *Cr, *Ci, *D, *z, *delta_bias;
  double* y;
} complex_problem;

static void scan_channel_complex(const complex_problem* p, int64_t b, int64_t d,
                                 double complex* h) {
  const int64_t L = p->L, N = p->N;
  const int64_t group = d / (p->dim / p->ngroups);
  const double* xr = p->x + (b * p->dim + d) * L;
  const double* dr = p->delta + (b * p->dim + d) * L;
  const int64_t goff = (b * p->ngroups + group) * N * L;
  const double* zr = p->z ? p->z + (b * p->dim + d) * L : NULL;
  double* yr = p->y + (b * p->dim + d) * L;
  const double bias = p->delta_bias ? p->delta_bias[d] : 0.0;
  const double Dd = p->D ? p->D[d] : 0.0;

  for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double v = dr[t] + bias;
    const double delta = p->delta_softplus ? softplus(v) : v;
    const double xt = xr[t];
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double complex a = p->Ar[d * N + n] + I * p->Ai[d * N + n];
      const double complex Bt = p->Br[goff + n * L + t] + I * p->Bi[goff + n * L + t];
      const double complex Ct = p->Cr[goff + n * L + t] + I * p->Ci[goff + n * L + t];
      const double complex Abar = cexp(delta * a);
      const double complex Bbar = delta * Bt;
      h[n] = Abar * h[n] + Bbar * xt;
      acc += creal(Ct * h[n]);
    }
    double yt = acc + Dd * xt;
    if (zr) yt *= silu(zr[t]);
    yr[t] = yt;
  }
}

typedef struct { const complex_problem* p; int64_t lo, hi; } complex_part;

static void* complex_worker(void* arg) {
  complex_part* w = (complex_part*)arg;
  double complex hbuf[1024];
  for (int64_t c = w->lo; c < w->hi; ++c)
    scan_channel_complex(w->p, c / w->p->dim, c % w->p->dim, hbuf);
  return NULL;
}

/* The complex-A scan for every (b, d) channel over nthreads threads; 0, or -1 on bad sizes. */
int ssm_oracle_scan_complex(int64_t batch, int64_t dim, int64_t L, int64_t N, int64_t ngroups,
                            int delta_softplus, const double* x, const double* delta,
                            const double* Ar, const double* Ai, const double* Br,
                            const double* Bi, const double* Cr, const double* Ci,
                            const double* D, const double* z, const double* delta_bias, double* y,
                            int nthreads) {
  if (batch < 0 || dim < 1 || L < 0 || N < 1 || N > 1024 || ngroups < 1 || dim % ngroups) return -1;
  if (!x || !delta || !Ar || !Ai || !Br || !Bi || !Cr || !Ci || !y) return -1;
  complex_problem p = {batch, dim, L, N, ngroups, delta_softplus, x, delta, Ar, Ai, Br, Bi,
                       Cr, Ci, D, z, delta_bias, y};
  const int64_t channels = batch * dim;
  if (channels == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > channels) nthreads = (int)channels;
  pthread_t th[256];
  complex_part parts[256];
  int started[256] = {0};
  const int64_t per = (channels + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    parts[t].p = &p;
    parts[t].lo = per * t;
    parts[t].hi = per * (t + 1) < channels ? per * (t + 1) : channels;
    if (parts[t].lo >= parts[t].hi) continue;
    if (nthreads == 1 || pthread_create(&th[t], NULL, complex_worker, &parts[t]) != 0)
      complex_worker(&parts[t]);
    else
      started[t] = 1;
  }
  for (int t = 0; t < nthreads; ++t) if (started[t]) pthread_join(th[t], NULL);
  return 0;
}
