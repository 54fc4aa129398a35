/*
 * FP64 CPU oracle for the gated delta rule (prompt-path DeltaNet recurrence) and the
 * gated RMS output norm.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code with the HIP library; the two meet only through the input arrays.
 *
 * Sources (web pages, cited by title and section):
 *   [PR413]  "#413 prefill: DeltaNet recurrence with the three value heads of a key head
 *            in one thread", sections "What changes" and "Exactness".
 *   [PR1372] "#1372 DeltaNet recurrence: STRATA_GDN_CHUNKED=1", section "What it does"
 *            and the accuracy table under "Measured".
 *
 * O1, the recurrence, per value head h (value head h reads key head h mod n_k_heads,
 * [PR413] "What changes": the heads that share a key head are h, h+16, h+32):
 *     a_t   = exp(g_t)                         (g is the log-decay, g <= 0)
 *     kv    = a_t * S_{t-1}^T k_t              (kv sum over the key dim)
 *     d     = beta_t * (v_t - kv)              (delta-rule correction)
 *     S_t   = a_t * S_{t-1} + k_t d^T          (rank-1 state update)
 *     o_t   = S_t^T q_t                        (output sum from the updated state)
 * S is dk x dv, row i = key dim, column j = value dim.  This is the definition itself,
 * evaluated in double precision from the same float32 inputs the GPU receives
 * ([PR1372] "Measured": accuracy is reported against an FP64 recurrence).
 *
 * O2, the output norm, per (token, value head) row of dv values:
 *     r = 1 / sqrt(mean_j o_j^2 + eps)
 *     y_j = fp16_round_nearest_even(o_j * r * w[h][j] * sigmoid(z_j))
 * [PR413] "What changes" names the norm and its FP16 copy y_h but prints no formula;
 * the gate is the sigmoid of z and the weight is per value head (the plainest reading
 * of a "gated RMS output norm"; parity of the gate form against the pages is unpinned).
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math, so the FP64 evaluation is
 * the plain IEEE one).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of O1 on one head: updates S in place and writes o_t. */
static void o1_token(double* S, const double* qt, const double* kt, const double* vt,
                     double gt, double bt, double* ot, int dk, int dv, double* kv) {
  const double a = exp(gt);
  for (int j = 0; j < dv; ++j) kv[j] = 0.0;
  for (int i = 0; i < dk; ++i) {
    const double ki = kt[i];
    const double* Si = S + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) kv[j] += Si[j] * ki;
  }
  /* kv now holds S_{t-1}^T k_t; the decay is applied to the state before the read. */
  for (int j = 0; j < dv; ++j) kv[j] = bt * (vt[j] - a * kv[j]); /* kv <- d */
  for (int i = 0; i < dk; ++i) {
    const double ki = kt[i];
    double* Si = S + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) Si[j] = a * Si[j] + ki * kv[j];
  }
  for (int j = 0; j < dv; ++j) ot[j] = 0.0;
  for (int i = 0; i < dk; ++i) {
    const double qi = qt[i];
    const double* Si = S + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) ot[j] += Si[j] * qi;
  }
}

/*
 * O1 over a list of value heads, reading float32 inputs in the library's layout:
 *   q, k       [T][n_k_heads][dk]      v   [T][n_v_heads][dv]
 *   g, beta    [T][n_v_heads]          state_in [n_v_heads][dk][dv]
 * For each selected head heads[s] it writes
 *   o_sel      [n_sel][T][dv]          state_sel [n_sel][dk][dv]      (double)
 * Heads are independent; OpenMP splits them over n_threads threads (<= 0: default).
 * Returns 0, or -1 on a bad argument.
 */
int gdn_oracle_recurrence(const float* q, const float* k, const float* v, const float* g,
                          const float* beta, const float* state_in, int64_t T,
                          int n_k_heads, int n_v_heads, int dk, int dv,
                          const int* heads, int n_sel, double* o_sel, double* state_sel,
                          int n_threads) {
  if (T < 0 || n_k_heads < 1 || n_v_heads < 1 || dk < 1 || dv < 1 || n_sel < 0) return -1;
  for (int s = 0; s < n_sel; ++s)
    if (heads[s] < 0 || heads[s] >= n_v_heads) return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < n_sel; ++s) {
    const int h = heads[s];
    const int kh = h % n_k_heads;
    double* S = state_sel + (size_t)s * dk * dv;
    double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * dk + 2 * dv));
    double* qt = buf;
    double* kt = buf + dk;
    double* vt = buf + 2 * dk;
    double* kv = buf + 2 * dk + dv;
    for (size_t e = 0; e < (size_t)dk * dv; ++e)
      S[e] = (double)state_in[(size_t)h * dk * dv + e];
    for (int64_t t = 0; t < T; ++t) {
      const float* qs = q + ((size_t)t * n_k_heads + kh) * dk;
      const float* ks = k + ((size_t)t * n_k_heads + kh) * dk;
      const float* vs = v + ((size_t)t * n_v_heads + h) * dv;
      for (int i = 0; i < dk; ++i) { qt[i] = qs[i]; kt[i] = ks[i]; }
      for (int j = 0; j < dv; ++j) vt[j] = vs[j];
      o1_token(S, qt, kt, vt, (double)g[(size_t)t * n_v_heads + h],
               (double)beta[(size_t)t * n_v_heads + h],
               o_sel + ((size_t)s * T + t) * dv, dk, dv, kv);
    }
    free(buf);
  }
  return 0;
}

/*
 * O1 for one head from double inputs (used by pins that need inputs not representable
 * in float32, e.g. a key renormalised in FP64):
 *   q, k [T][dk]   v [T][dv]   g, beta [T]   state [dk][dv] (in: S0, out: S_T)   o [T][dv]
 */
int gdn_oracle_recurrence_f64(const double* q, const double* k, const double* v,
                              const double* g, const double* beta, double* state,
                              int64_t T, int dk, int dv, double* o) {
  if (T < 0 || dk < 1 || dv < 1) return -1;
  double* kv = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int64_t t = 0; t < T; ++t)
    o1_token(state, q + (size_t)t * dk, k + (size_t)t * dk, v + (size_t)t * dv, g[t], beta[t],
             o + (size_t)t * dv, dk, dv, kv);
  free(kv);
  return 0;
}

/*
 * IEEE binary16 encoding of a double, rounded to nearest, ties to even, with gradual
 * underflow and overflow to infinity.  Written from the binary16 format definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).
 */
uint16_t gdn_oracle_f64_to_f16(double x) {
  uint64_t bits;
  memcpy(&bits, &x, sizeof bits);
  const uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
  const int ebits = (int)((bits >> 52) & 0x7ff);
  const uint64_t frac = bits & ((1ull << 52) - 1);
  if (ebits == 0x7ff) return (uint16_t)(sign | (frac ? 0x7e00u : 0x7c00u));
  if (ebits == 0) return sign; /* zero or a double subnormal: far below half's range */
  const int e = ebits - 1023;          /* x = m * 2^(e-52), m has 53 bits */
  const uint64_t m = frac | (1ull << 52);
  int he = e + 15;                     /* biased half exponent if normal */
  if (he >= 1) {
    uint64_t qv = m >> 42;             /* 11 significant bits */
    const uint64_t rem = m & ((1ull << 42) - 1);
    const uint64_t halfway = 1ull << 41;
    if (rem > halfway || (rem == halfway && (qv & 1))) ++qv;
    if (qv == (1ull << 11)) { qv >>= 1; ++he; }
    if (he >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(he << 10) | (uint16_t)(qv & 0x3ff));
  }
  /* subnormal half: count units of 2^-24, i.e. x / 2^-24 = m * 2^(e-28) */
  const int shift = 28 - e;            /* >= 43 here */
  if (shift >= 54) return sign;        /* below half of 2^-24 */
  uint64_t qv = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (qv & 1))) ++qv;
  return (uint16_t)(sign | (uint16_t)qv); /* qv == 1024 encodes the smallest normal */
}

/*
 * O2 over n_rows rows of dv values:
 *   o, z   [n_rows][dv]  double      w [n_w][dv] double     w_idx [n_rows] (row -> w row)
 *   y64    [n_rows][dv]  double      (the value before rounding; may be NULL)
 *   y16    [n_rows][dv]  uint16      (IEEE binary16 bits)
 */
int gdn_oracle_out_norm(const double* o, const double* z, const double* w, const int* w_idx,
                        double eps, int64_t n_rows, int n_w, int dv, double* y64,
                        uint16_t* y16, int n_threads) {
  if (n_rows < 0 || dv < 1 || n_w < 1) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (w_idx[r] < 0 || w_idx[r] >= n_w) return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    const double* orow = o + (size_t)r * dv;
    const double* zrow = z + (size_t)r * dv;
    const double* wrow = w + (size_t)w_idx[r] * dv;
    double ss = 0.0;
    for (int j = 0; j < dv; ++j) ss += orow[j] * orow[j];
    const double rs = 1.0 / sqrt(ss / dv + eps);
    for (int j = 0; j < dv; ++j) {
      const double gate = 1.0 / (1.0 + exp(-zrow[j]));
      const double val = orow[j] * rs * wrow[j] * gate;
      if (y64) y64[(size_t)r * dv + j] = val;
      y16[(size_t)r * dv + j] = gdn_oracle_f64_to_f16(val);
    }
  }
  return 0;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * O3, the step before the recurrence ("Round 20 Track C Audit: gdn_pre ...", section 1,
 * the key-head branch of gdn_pre and its helper gp_conv; section 2 lists its outputs: the
 * normalised q and k, the convolved v, the gate and beta, and the conv history).
 *
 * x is the projection output [T][C] with C = 2*Hk*dk + Hv*dv channels per token: the q
 * channels of key head kh at kh*dk, the k channels of key head kh at (Hk + kh)*dk, the v
 * channels of value head h at 2*Hk*dk + h*dv (the page's key-head branch addresses q at
 * kh*S and k at (hk_n + kh)*S within a token's row).  Per token t and channel c:
 *
 *   xe      = the 3 history rows (the conv inputs of the 3 tokens before the call, oldest
 *             first) followed by the T rows of x
 *   u[t][c] = sum_{j=0..3} w[c][j] * xe[t + j][c]    (4-tap causal conv: the page loads
 *             the four taps of a channel as one float4 and applies them to the rows at
 *             t-3, t-2, t-1, t; tap 3 multiplies the current token)
 *   u       = act(u)   (activation == 1: SiLU, u / (1 + e^-u); activation == 0: none.
 *             The page does not name the activation: a reading, parity unpinned)
 *   q[t][kh][i] = u_q[i] / sqrt(sum_i u_q[i]^2 + eps) / sqrt(dk)
 *   k[t][kh][i] = u_k[i] / sqrt(sum_i u_k[i]^2 + eps)
 *             (L2 normalisation over the head's dk channels; the q scale 1/sqrt(dk) of the
 *             workload's q.  The form of eps is a reading, parity unpinned)
 *   v[t][h][j]  = u_v[j]
 *   hist_out[j] = xe[T + j], j = 0, 1, 2   (the conv inputs of the call's last 3 tokens,
 *             taken from hist_in where the call has fewer than 3 tokens)
 *   g[t][h]     = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
 *   beta[t][h]  = 1 / (1 + exp(-b[t][h]))
 *             (the page prints no gate or beta formula: the common gated-DeltaNet form is
 *             taken as a reading, parity unpinned; it gives g < 0 and beta in (0, 1))
 *
 * Inputs are float32 (the arrays the GPU receives) and widened to double; outputs are
 * double.  a, b, A_log, dt_bias, g and beta may all be NULL (no gate and beta).
 * Returns 0, or -1 on a bad argument.
 */
static double softplus_f64(double z) {
  return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z)); /* log(1 + e^z), both branches exact */
}

int gdn_oracle_pre(const float* x, const float* w, const float* hist_in, const float* a,
                   const float* b, const float* A_log, const float* dt_bias, int activation,
                   double eps, int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                   double* q, double* k, double* v, double* g, double* beta,
                   double* hist_out) {
  if (T < 0 || n_k_heads < 1 || n_v_heads < 1 || dk < 1 || dv < 1) return -1;
  if (activation != 0 && activation != 1) return -1;
  const int gates = a != NULL;
  if (gates && (!b || !A_log || !dt_bias || !g || !beta)) return -1;
  const int64_t C = 2 * (int64_t)n_k_heads * dk + (int64_t)n_v_heads * dv;
  double* u = (double*)malloc(sizeof(double) * (size_t)C);
  for (int64_t t = 0; t < T; ++t) {
    /* the conv over the extended sequence, then the activation */
    for (int64_t c = 0; c < C; ++c) {
      double s = 0.0;
      for (int j = 0; j < 4; ++j) {
        const int64_t r = t + j; /* row of xe */
        const double xv = r < 3 ? (double)hist_in[r * C + c] : (double)x[(r - 3) * C + c];
        s += (double)w[c * 4 + j] * xv;
      }
      u[c] = activation ? s / (1.0 + exp(-s)) : s;
    }
    /* q and k: L2 normalisation per key head, q also scaled by 1/sqrt(dk) */
    for (int kh = 0; kh < n_k_heads; ++kh) {
      const double* uq = u + (int64_t)kh * dk;
      const double* uk = u + ((int64_t)n_k_heads + kh) * dk;
      double sq = 0.0, sk = 0.0;
      for (int i = 0; i < dk; ++i) {
        sq += uq[i] * uq[i];
        sk += uk[i] * uk[i];
      }
      const double rq = 1.0 / sqrt(sq + eps) / sqrt((double)dk);
      const double rk = 1.0 / sqrt(sk + eps);
      double* qo = q + (t * n_k_heads + kh) * dk;
      double* ko = k + (t * n_k_heads + kh) * dk;
      for (int i = 0; i < dk; ++i) {
        qo[i] = uq[i] * rq;
        ko[i] = uk[i] * rk;
      }
    }
    for (int h = 0; h < n_v_heads; ++h) {
      const double* uv = u + 2 * (int64_t)n_k_heads * dk + (int64_t)h * dv;
      double* vo = v + (t * n_v_heads + h) * dv;
      for (int j = 0; j < dv; ++j) vo[j] = uv[j];
    }
    if (gates) {
      for (int h = 0; h < n_v_heads; ++h) {
        const int64_t e = t * n_v_heads + h;
        g[e] = -exp((double)A_log[h]) * softplus_f64((double)a[e] + (double)dt_bias[h]);
        beta[e] = 1.0 / (1.0 + exp(-(double)b[e]));
      }
    }
  }
  /* the conv inputs of the last 3 rows of xe */
  for (int j = 0; j < 3; ++j) {
    const int64_t r = T + j;
    for (int64_t c = 0; c < C; ++c)
      hist_out[j * C + c] = r < 3 ? (double)hist_in[r * C + c] : (double)x[(r - 3) * C + c];
  }
  free(u);
  return 0;
}
