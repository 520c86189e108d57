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
 *     h_n  = a * h_n + k_t * B[b, g, n, t] * u[b, d, t]
 *            k_t = dt_t (exponential-Euler), or (a - 1) / A with zero-order hold
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
  int32_t zoh;              /* 1: zero-order-hold input coefficient (see in_coef) */
  int32_t trap;             /* 1: exponential-trapezoidal rule (see run_row) */
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

/* The input coefficient of the discretisation: dt (exponential-Euler, Bbar = dt B), or with
 * zero-order hold Bbar = (dt A)^-1 (exp(dt A) - 1) dt B = (exp(dt A) - 1) / A B, whose limit
 * at A = 0 is dt B (omica.com.cn explainer, sections 3 and 5). */
static double in_coef(const sso_problem* p, double dt, double an) {
  if (!p->zoh || an == 0.0) return dt;
  return expm1(dt * an) / an;
}

typedef struct {
  const sso_problem* p;
  const int64_t* rows;
  int64_t nrows;
  double* y;
  double* h_final;
  int tid, nthreads;
  int status;
} job_t;

/* The exponential-trapezoidal rule (omica.com.cn explainer, section 6.3, the recurrence of
 * Mamba-3) averages the input of the current and the previous step:
 *   h_t = a_t h_{t-1} + 1/2 (e_t + a_t e_{t-1}),   e_t = k_t B_t u_t  (k_t the input coefficient),
 * with nothing before the first step.  The state passed in and out of a call (h0, h_final) is
 * h + 1/2 e of the step before / the last step, the quantity that carries the rule across a
 * boundary (it lets a sequence be scanned in pieces); run_row keeps h and the previous e. */
static void run_row(const sso_problem* p, int64_t row, int64_t out_index, double* h, double* y,
                    double* h_final) {
  const int64_t L = p->length, N = p->nstate, Dc = p->channels;
  const int64_t b = row / Dc, d = row % Dc;
  const int64_t hd = d / (Dc / p->heads);
  const int64_t g = d / (Dc / p->groups);
  const int64_t urow = (b * Dc + d) * L;
  const int64_t drow = (b * p->heads + hd) * L;
  const int64_t bcrow = (b * p->groups + g) * N * L;
  /* h[n]: the state; h[N + n]: the previous step's input term e (trapezoidal rule only) */
  for (int64_t n = 0; n < N; ++n) {
    h[n] = p->h0 ? p->h0[out_index * N + n] : 0.0;
    h[N + n] = 0.0;
  }
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
      const double e = in_coef(p, dt, an) * bn * ut;
      if (p->trap) {
        h[n] = a * h[n] + 0.5 * (e + a * h[N + n]);
        h[N + n] = e;
      } else {
        h[n] = a * h[n] + e;
      }
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
    for (int64_t n = 0; n < N; ++n) h_final[out_index * N + n] = h[n] + (p->trap ? 0.5 * h[N + n] : 0.0);
}

static void* worker(void* arg) {
  job_t* j = (job_t*)arg;
  double* h = (double*)malloc(sizeof(double) * (size_t)(j->p->nstate > 0 ? 2 * j->p->nstate : 1));
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

/* ------------------------------------------------------------------------------------------ */
/* Backward (reverse-mode gradient) of the same recurrence, in float64.
 *
 * Given dy = dLoss/dy, the gradients of every input follow from the forward definition above by
 * the chain rule, taken step by step in reverse time order (the pages describe training that
 * recomputes the states instead of storing them -- bqwf.cn survey, section 2.2 -- but name no
 * formula; this is the plain derivative).  With s(z) = z sigmoid(z) and y0_t the output before
 * the gate:
 *
 *   dy0_t    = dy_t s(z_t)                      dz_t = dy_t y0_t s'(z_t)
 *   g_{t,n}  = C_{t,n} dy0_t + a_{t+1,n} g_{t+1,n}        (dLoss/dh_{t,n}; g after the end = 0)
 *   dC_{t,n} += dy0_t h_{t,n}                   dB_{t,n} += g_{t,n} dt_t u_t
 *   du_t     = dy0_t D + sum_n g_{t,n} dt_t B_{t,n}       dD += dy0_t u_t
 *   ddt_t    = sum_n g_{t,n} (h_{t-1,n} a_{t,n} A_n + B_{t,n} u_t)
 *   dA_n    += sum_t g_{t,n} h_{t-1,n} a_{t,n} dt_t
 *   dx_t     = ddt_t sigmoid(x_t)  (softplus' ; dx_t = ddt_t without softplus)
 *   ddelta_t += dx_t                            dbias += dx_t
 *   dh0_n    = a_{0,n} g_{0,n}                  (gradient of the initial state)
 *
 * B, C, A (scalar per head), D (per head), delta and delta_bias are shared between rows; their
 * gradients are sums over the rows that use them.  Each thread sums its rows into a private
 * buffer; the buffers are added in thread order at the end (deterministic).
 */

typedef struct {
  double* du;      /* [batch, channels, L] */
  double* ddelta;  /* [batch, heads, L] */
  double* dA;      /* [channels, N] or [heads] */
  double* dB;      /* [batch, groups, N, L] */
  double* dC;      /* [batch, groups, N, L] */
  double* dD;      /* [channels] or [heads], or NULL */
  double* dz;      /* [batch, channels, L], or NULL */
  double* dbias;   /* [heads], or NULL */
  double* dh0;     /* [batch * channels, N], or NULL */
} sso_grads;

typedef struct {
  const sso_problem* p;
  const double* dy;
  sso_grads out;       /* shared, per-row outputs (du, dz, dh0) */
  sso_grads part;      /* this thread's sums (ddelta, dA, dB, dC, dD, dbias) */
  int tid, nthreads;
  int status;
} bjob_t;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static void bwd_row(const sso_problem* p, const double* dy, int64_t row, double* hs, double* gcur,
                    const sso_grads* out, const sso_grads* part) {
  const int64_t L = p->length, N = p->nstate, Dc = p->channels;
  const int64_t b = row / Dc, d = row % Dc;
  const int64_t hd = d / (Dc / p->heads);
  const int64_t g = d / (Dc / p->groups);
  const int64_t urow = (b * Dc + d) * L;
  const int64_t drow = (b * p->heads + hd) * L;
  const int64_t bcrow = (b * p->groups + g) * N * L;
  const double bias = p->delta_bias ? p->delta_bias[hd] : 0.0;
  const double dskip = p->D ? p->D[p->d_per_head ? hd : d] : 0.0;
  /* forward, keeping every state: hs[t + 1][n] = h_{t,n}, hs[0] = initial state */
  for (int64_t n = 0; n < N; ++n) hs[n] = p->h0 ? p->h0[row * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double x = load(p->delta, p->in_dtype, drow + t) + bias;
    const double dt = p->softplus ? softplus(x) : x;
    const double ut = load(p->u, p->in_dtype, urow + t);
    for (int64_t n = 0; n < N; ++n) {
      const double an = p->a_per_head ? p->A[hd] : p->A[d * N + n];
      const double bn = load(p->B, p->in_dtype, bcrow + n * L + t);
      hs[(t + 1) * N + n] = exp(dt * an) * hs[t * N + n] + dt * bn * ut;
    }
  }
  /* reverse: gcur[n] holds a_{t+1,n} g_{t+1,n} entering step t */
  for (int64_t n = 0; n < N; ++n) gcur[n] = 0.0;
  for (int64_t t = L - 1; t >= 0; --t) {
    const double x = load(p->delta, p->in_dtype, drow + t) + bias;
    const double dt = p->softplus ? softplus(x) : x;
    const double ut = load(p->u, p->in_dtype, urow + t);
    double y0 = dskip * ut;
    for (int64_t n = 0; n < N; ++n) y0 += load(p->C, p->in_dtype, bcrow + n * L + t) * hs[(t + 1) * N + n];
    double dy0 = dy[row * L + t];
    if (p->z) {
      const double zt = load(p->z, p->in_dtype, urow + t);
      const double sg = sigmoid(zt);
      if (out->dz) out->dz[row * L + t] = dy0 * y0 * sg * (1.0 + zt * (1.0 - sg));
      dy0 *= zt * sg;
    }
    double du = dy0 * dskip, ddt = 0.0;
    if (part->dD) part->dD[p->d_per_head ? hd : d] += dy0 * ut;
    for (int64_t n = 0; n < N; ++n) {
      const double an = p->a_per_head ? p->A[hd] : p->A[d * N + n];
      const double a = exp(dt * an);
      const double bn = load(p->B, p->in_dtype, bcrow + n * L + t);
      const double cn = load(p->C, p->in_dtype, bcrow + n * L + t);
      const double gn = cn * dy0 + gcur[n];
      const double hprev = hs[t * N + n];
      part->dC[bcrow + n * L + t] += dy0 * hs[(t + 1) * N + n];
      part->dB[bcrow + n * L + t] += gn * dt * ut;
      du += gn * dt * bn;
      ddt += gn * (hprev * a * an + bn * ut);
      part->dA[p->a_per_head ? hd : d * N + n] += gn * hprev * a * dt;
      gcur[n] = a * gn;
    }
    out->du[row * L + t] = du;
    const double dx = p->softplus ? ddt * sigmoid(x) : ddt;
    part->ddelta[drow + t] += dx;
    if (part->dbias) part->dbias[hd] += dx;
  }
  if (out->dh0)
    for (int64_t n = 0; n < N; ++n) out->dh0[row * N + n] = gcur[n];
}

static int64_t grad_sizes(const sso_problem* p, int64_t* n_delta, int64_t* n_A, int64_t* n_BC, int64_t* n_D) {
  *n_delta = p->batch * p->heads * p->length;
  *n_A = p->a_per_head ? p->heads : p->channels * p->nstate;
  *n_BC = p->batch * p->groups * p->nstate * p->length;
  *n_D = p->d_per_head ? p->heads : p->channels;
  return *n_delta + *n_A + 2 * *n_BC + *n_D + p->heads;
}

static void* bworker(void* arg) {
  bjob_t* j = (bjob_t*)arg;
  const sso_problem* p = j->p;
  const int64_t N = p->nstate, L = p->length;
  double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * (N > 0 ? N : 1)));
  double* gcur = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  if (!hs || !gcur) {
    free(hs);
    free(gcur);
    j->status = -1;
    return NULL;
  }
  const int64_t total = p->batch * p->channels;
  for (int64_t row = j->tid; row < total; row += j->nthreads) bwd_row(p, j->dy, row, hs, gcur, &j->out, &j->part);
  free(hs);
  free(gcur);
  j->status = 0;
  return NULL;
}

/* Gradients of sum(dy * y) with respect to every input, for all rows.  dy: [batch, channels, L]
 * float64.  Outputs (float64, overwritten): du, ddelta, dA, dB, dC required; dD, dz, dbias, dh0
 * optional (NULL: not computed).  Returns 0, or -1 on a bad argument or allocation failure. */
int sso_scan_bwd(const sso_problem* p, const double* dy, sso_grads* g, int nthreads) {
  if (!p || !dy || !g || !g->du || !g->ddelta || !g->dA || !g->dB || !g->dC) return -1;
  if (p->zoh || p->trap) return -1; /* the backward is derived for the exponential-Euler rule */
  if (!p->u || !p->delta || !p->A || !p->B || !p->C) return -1;
  if (p->channels <= 0 || p->heads <= 0 || p->groups <= 0 || p->channels % p->heads ||
      p->channels % p->groups || p->nstate < 0 || p->length < 0 || p->batch < 0)
    return -1;
  int64_t n_delta, n_A, n_BC, n_D;
  const int64_t nsum = grad_sizes(p, &n_delta, &n_A, &n_BC, &n_D);
  const int64_t total = p->batch * p->channels;
  memset(g->du, 0, sizeof(double) * (size_t)(total * p->length));
  memset(g->ddelta, 0, sizeof(double) * (size_t)n_delta);
  memset(g->dA, 0, sizeof(double) * (size_t)n_A);
  memset(g->dB, 0, sizeof(double) * (size_t)n_BC);
  memset(g->dC, 0, sizeof(double) * (size_t)n_BC);
  if (g->dD) memset(g->dD, 0, sizeof(double) * (size_t)n_D);
  if (g->dz) memset(g->dz, 0, sizeof(double) * (size_t)(total * p->length));
  if (g->dbias) memset(g->dbias, 0, sizeof(double) * (size_t)p->heads);
  if (g->dh0) memset(g->dh0, 0, sizeof(double) * (size_t)(total * p->nstate));
  if (total == 0 || p->length == 0) return 0;  /* no steps: every gradient is zero */
  if (nthreads < 1) nthreads = 1;
  if (nthreads > total) nthreads = (int)total;
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  bjob_t* jobs = (bjob_t*)calloc((size_t)nthreads, sizeof(bjob_t));
  double* sums = (double*)calloc((size_t)(nthreads * nsum), sizeof(double));
  if (!th || !jobs || !sums) {
    free(th);
    free(jobs);
    free(sums);
    return -1;
  }
  for (int i = 0; i < nthreads; ++i) {
    double* s = sums + (int64_t)i * nsum;
    sso_grads part = {NULL, s, s + n_delta, s + n_delta + n_A, s + n_delta + n_A + n_BC,
                      s + n_delta + n_A + 2 * n_BC, NULL, s + n_delta + n_A + 2 * n_BC + n_D, NULL};
    if (!g->dD) part.dD = NULL;
    if (!g->dbias) part.dbias = NULL;
    jobs[i] = (bjob_t){p, dy, *g, part, i, nthreads, -1};
    if (pthread_create(&th[i], NULL, bworker, &jobs[i]) != 0) {
      bworker(&jobs[i]);
      th[i] = 0;
    }
  }
  int rc = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (th[i]) pthread_join(th[i], NULL);
    if (jobs[i].status != 0) rc = -1;
  }
  for (int i = 0; i < nthreads && rc == 0; ++i) {
    const sso_grads* s = &jobs[i].part;
    for (int64_t k = 0; k < n_delta; ++k) g->ddelta[k] += s->ddelta[k];
    for (int64_t k = 0; k < n_A; ++k) g->dA[k] += s->dA[k];
    for (int64_t k = 0; k < n_BC; ++k) g->dB[k] += s->dB[k];
    for (int64_t k = 0; k < n_BC; ++k) g->dC[k] += s->dC[k];
    if (g->dD)
      for (int64_t k = 0; k < n_D; ++k) g->dD[k] += s->dD[k];
    if (g->dbias)
      for (int64_t k = 0; k < p->heads; ++k) g->dbias[k] += s->dbias[k];
  }
  free(th);
  free(jobs);
  free(sums);
  return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* Causal depthwise convolution in front of the scan (each Mamba block has a causal 1-D
 * convolution that adds local context before the selective SSM: bqwf.cn survey, section 3.1;
 * the decoding state then keeps the last few inputs: study notes, pitfalls).  Per (b, d):
 *
 *   out_t = bias_d + sum_{j=0}^{W-1} w[d, j] * x_{t - (W-1) + j}      (w[d, W-1] on the newest)
 *   out_t = out_t * sigmoid(out_t)                                    (if silu)
 *
 * with x_{-W+1..-1} from `state` ([rows, W-1], oldest first) or zero; the last W-1 inputs are
 * returned in `state_out`.  x: [batch, channels, L] (dtype as in sso_problem), w: [channels, W],
 * out: [batch, channels, L] float64. */
int sso_conv1d(int64_t batch, int64_t channels, int64_t L, int32_t dtype, const void* x, const double* w,
               int64_t W, const double* bias, const double* state, int32_t silu, double* out, double* state_out) {
  if (!x || !w || !out || W < 1 || batch < 0 || channels < 0 || L < 0) return -1;
  for (int64_t r = 0; r < batch * channels; ++r) {
    const int64_t d = r % channels;
    for (int64_t t = 0; t < L; ++t) {
      double acc = bias ? bias[d] : 0.0;
      for (int64_t j = 0; j < W; ++j) {
        const int64_t s = t - (W - 1) + j;
        double xv = 0.0;
        if (s >= 0) xv = load(x, dtype, r * L + s);
        else if (state) xv = state[r * (W - 1) + (W - 1) + s];   /* s = -(W-1) .. -1 */
        acc += w[d * W + j] * xv;
      }
      if (silu) acc = acc / (1.0 + exp(-acc));
      out[r * L + t] = acc;
    }
    if (state_out)
      for (int64_t j = 0; j < W - 1; ++j) {
        const int64_t s = L - (W - 1) + j;
        state_out[r * (W - 1) + j] = s >= 0 ? load(x, dtype, r * L + s)
                                            : (state ? state[r * (W - 1) + (W - 1) + s] : 0.0);
      }
  }
  return 0;
}
