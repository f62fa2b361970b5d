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
