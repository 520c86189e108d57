/*
 * ss_oracle.c -- CPU oracle for the selective-scan forward (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this file:
 * it exists so that tests, the smoke check and the benchmark's CPU baseline can
 * check the GPU kernels against a plain, slow, obviously correct definition.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, per batch b and channel d, sequentially over t, in float64:
 *
 *   x_t    = delta[b, hd, t] + delta_bias[hd]              (bias optional)
 *   dt_t   = softplus(x_t) = log(1 + exp(x_t))             (if enabled; else dt_t = x_t)
 *   for each state n:
 *     a    = exp(dt_t * A[d, n])                           (A[hd] in the scalar-decay layout)
 *     h_n  = a * h_n + dt_t * B[b, g, n, t] * u[b, d, t]
 *   y_t    = sum_n C[b, g, n, t] * h_n + D * u[b, d, t]    (D optional)
 *   y_t   *= z_t / (1 + exp(-z_t))                         (gate optional, z = z[b, d, t])
 *
 * with h_n = 0 before t = 0 unless an initial state is passed.  hd = d / (channels / heads)
 * is the head (hd = d when delta is per channel); g = d / (channels / groups) is the B/C group.
 *
 * Sources, by page:
 *  - The recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t, y_t = C_t h_t and the input-dependent
 *    B_t, C_t, Delta_t = softplus(Linear(x_t)): omica.com.cn Mamba explainer (news 823493),
 *    section 3 (the mathematics of the state) and section 5 (selection mechanism).
 *  - Abar = exp(Delta A), Bbar = Delta B (exponential-Euler, which that explainer's section 6.3
 *    attributes to Mamba-1 and Mamba-2); the same Delta*B*x_t update appears in the one-step
 *    pseudocode of the "Mamba -- selective state space model" study notes (estelledc.github.io),
 *    case 1.
 *  - The optional D*x feed-through: explainer section 3 (output equation; the page calls the term usually dropped).
 *  - Scalar decay per head (A_t = alpha_t I): bqwf.cn state-space survey (news 437117), section 3.2.
 *  - The gate after the SSM: juejin.cn post on Mamba's history, section 2 (first-generation
 *    Mamba), whose block replaces attention by a selective SSM followed by gating.  The pages
 *    give no formula; the gate is read as y * silu(z), silu(z) = z * sigmoid(z).
 *  Softplus is evaluated as max(x, 0) + log1p(exp(-|x|)), which equals log(1 + e^x) exactly
 *  in real arithmetic and avoids overflow.
 *
 * Build: gcc -O2 -fPIC -shared -pthread (no -ffast-math), libm exp/log1p in double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { SSO_F32 = 0, SSO_BF16 = 1, SSO_F64 = 2 };

typedef struct {
  int64_t batch, channels, length, nstate, groups, heads;
  int32_t in_dtype;   /* dtype of u, delta, B, C, z */
  int32_t a_per_head; /* 1: A is [heads]; 0: A is [channels, nstate] */
  int32_t d_per_head; /* 1: D is [heads]; 0: D is [channels] */
  int32_t softplus;   /* 1: dt = softplus(delta + bias) */
  const void* u;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;            /* NULL: no gate */
  const double* A;
  const double* D;          /* NULL: no feed-through */
  const double* delta_bias; /* NULL: no bias */
  const double* h0;         /* [nrows, nstate] initial state, NULL: zeros */
} sso_problem;

static double load(const void* p, int32_t dt, int64_t i) {
  if (dt == SSO_F64) return ((const double*)p)[i];
  if (dt == SSO_F32) return (double)((const float*)p)[i];
  /* bf16: the 16 bits are the high half of a float32 */
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

typedef struct {
  const sso_problem* p;
  const int64_t* rows;
  int64_t nrows;
  double* y;
  double* h_final;
  int tid, nthreads;
  int status;
} job_t;

static void run_row(const sso_problem* p, int64_t row, int64_t out_index, double* h, double* y,
                    double* h_final) {
  const int64_t L = p->length, N = p->nstate, Dc = p->channels;
  const int64_t b = row / Dc, d = row % Dc;
  const int64_t hd = d / (Dc / p->heads);
  const int64_t g = d / (Dc / p->groups);
  const int64_t urow = (b * Dc + d) * L;
  const int64_t drow = (b * p->heads + hd) * L;
  const int64_t bcrow = (b * p->groups + g) * N * L;
  for (int64_t n = 0; n < N; ++n) h[n] = p->h0 ? p->h0[out_index * N + n] : 0.0;
  const double bias = p->delta_bias ? p->delta_bias[hd] : 0.0;
  const double dskip = p->D ? p->D[p->d_per_head ? hd : d] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double x = load(p->delta, p->in_dtype, drow + t) + bias;
    const double dt = p->softplus ? softplus(x) : x;
    const double ut = load(p->u, p->in_dtype, urow + t);
    double yt = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double an = p->a_per_head ? p->A[hd] : p->A[d * N + n];
      const double a = exp(dt * an);
      const double bn = load(p->B, p->in_dtype, bcrow + n * L + t);
      const double cn = load(p->C, p->in_dtype, bcrow + n * L + t);
      h[n] = a * h[n] + dt * bn * ut;
      yt += cn * h[n];
    }
    if (p->D) yt += dskip * ut;
    if (p->z) {
      const double zt = load(p->z, p->in_dtype, urow + t);
      yt *= zt / (1.0 + exp(-zt));
    }
    y[out_index * L + t] = yt;
  }
  if (h_final)
    for (int64_t n = 0; n < N; ++n) h_final[out_index * N + n] = h[n];
}

static void* worker(void* arg) {
  job_t* j = (job_t*)arg;
  double* h = (double*)malloc(sizeof(double) * (size_t)(j->p->nstate > 0 ? j->p->nstate : 1));
  if (!h) {
    j->status = -1;
    return NULL;
  }
  for (int64_t i = j->tid; i < j->nrows; i += j->nthreads) {
    const int64_t row = j->rows ? j->rows[i] : i;
    run_row(j->p, row, i, h, j->y, j->h_final);
  }
  free(h);
  j->status = 0;
  return NULL;
}

/* Runs the recurrence for the listed rows (row = b * channels + d; NULL = all rows in order).
 * y: [nrows, length] float64.  h_final: [nrows, nstate] or NULL.  Returns 0, or -1 on a bad
 * argument or allocation failure. */
int sso_scan_fwd(const sso_problem* p, const int64_t* rows, int64_t nrows, double* y,
                 double* h_final, int nthreads) {
  if (!p || !y || !p->u || !p->delta || !p->A || !p->B || !p->C) return -1;
  if (p->channels <= 0 || p->heads <= 0 || p->groups <= 0 || p->channels % p->heads ||
      p->channels % p->groups || p->nstate < 0 || p->length < 0 || p->batch < 0)
    return -1;
  const int64_t total = p->batch * p->channels;
  if (!rows) nrows = total;
  for (int64_t i = 0; rows && i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= total) return -1;
  if (nrows == 0 || p->length == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nrows) nthreads = (int)nrows;
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  if (!th || !jobs) {
    free(th);
    free(jobs);
    return -1;
  }
  int rc = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (job_t){p, rows, nrows, y, h_final, i, nthreads, -1};
    if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) {
      worker(&jobs[i]); /* run inline if a thread cannot be created */
      th[i] = 0;
    }
  }
  for (int i = 0; i < nthreads; ++i) {
    if (th[i]) pthread_join(th[i], NULL);
    if (jobs[i].status != 0) rc = -1;
  }
  free(th);
  free(jobs);
  return rc;
}
