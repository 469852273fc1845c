/*
 * gdn_oracle.c -- plain, slow CPU oracle for the Gated DeltaNet layer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or helper with the GPU library; both sides are written independently from
 * the definitions below.
 *
 * Everything is double precision, token by token, in the order the
 * definitions state, with no blocking and no chunking.  Work is split over
 * independent heads / channels / rows with OpenMP; every reduction over
 * tokens or rows is done in a fixed order so results do not depend on the
 * thread count.
 *
 * Sources (page title, then section):
 *  - miles PR "port Qwen3.5 / Qwen3-Next GDN to the head-sharded layer":
 *    "What" (GDN as a linear-attention family on the shared layer; q/k/v and
 *    the conv are the channel-laid-out tensors), "Summary of an earlier run"
 *    (grouped-value heads: native GVA equals repeating q/k).
 *  - prime-rl PR "Qwen3.8 Flash Next ... layers/": "Summary" (the layer takes
 *    "silu"/"sigmoid" activation kwargs; ZeroCenteredRMSNorm; causal_conv1d
 *    with cu_seqlens; initial_state=None, output_final_state=False),
 *    "What I ran" (the three reference ops: conv, gated delta rule, gated
 *    norm).
 *  - Megatron-LM PR "Support gated delta net for Qwen3-Next (1/4)": GDN
 *    arguments (conv kernel 4, key/value head dim 128, 16 key heads),
 *    "--apply-layernorm-1p" (zero-centred RMSNorm), and the review comment
 *    that A_log stores log(A) and the forward uses exp(A_log).
 *
 * The pages never print the recurrence.  It is taken as the standard gated
 * delta rule of Gated DeltaNet:
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t (scale * q_t),
 * with S a d_v x d_k matrix per (sequence, value head).
 *
 * Readings where the pages are silent (each one is a choice):
 *  - conv: depthwise cross-correlation, taps w[c][0..K-1], w[c][K-1] on the
 *    current token, zero left padding at every sequence start, no bias,
 *    no state carried in or out; SiLU on every channel afterwards.
 *  - L2 normalisation of q and k per (token, head) over d_k:
 *    q_hat = a / sqrt(sum a^2 + eps).
 *  - gate: g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b),
 *    softplus computed exactly (no threshold).
 *  - grouped values: value head h reads key head h / (Hv / Hk).
 *  - gated norm: y = o * rsqrt(mean(o^2) + eps) * (1 + w) * act(z), w shared
 *    by all value heads, act = SiLU or sigmoid.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR 1

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), written so that it never overflows. */
static double softplus(double x) { return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* ---------------------------------------------------------------------------
 * Depthwise causal short convolution + SiLU + per-head L2 normalisation.
 *
 * x, y: [T][C] (row stride C).  w: [C][K].  cu: [N+1] token offsets.
 * Channels [0, n_l2) are L2-normalised in consecutive groups of dk (the q
 * block then the k block); channels [n_l2, C) (values) are not.
 * ------------------------------------------------------------------------- */
static void conv_silu_row(int64_t t, int64_t t0, int32_t C, int32_t K, const double* x,
                          const double* w, double* u, double* a) {
  for (int32_t c = 0; c < C; ++c) {
    double acc = 0.0;
    for (int32_t j = 0; j < K; ++j) {
      int64_t s = t - (K - 1) + j;   /* tap j reads token t-(K-1)+j */
      if (s >= t0) acc += w[(int64_t)c * K + j] * x[s * C + c];
    }
    u[c] = acc;
    a[c] = acc * sigm(acc);
  }
}

int oracle_conv_fwd(int64_t T, int32_t C, int32_t K, const double* x, const double* w,
                    const int32_t* cu, int32_t N, int32_t n_l2, int32_t dk, double eps,
                    double* y) {
  if (T < 0 || C <= 0 || K <= 0 || N < 0 || n_l2 < 0 || n_l2 > C || (n_l2 && (dk <= 0 || n_l2 % dk)))
    return OR_ERR;
  for (int32_t n = 0; n < N; ++n) {
    int64_t t0 = cu[n], t1 = cu[n + 1];
#pragma omp parallel for schedule(static)
    for (int64_t t = t0; t < t1; ++t) {
      double* u = (double*)malloc(sizeof(double) * C);
      double* a = (double*)malloc(sizeof(double) * C);
      conv_silu_row(t, t0, C, K, x, w, u, a);
      for (int32_t c = 0; c < C; ++c) y[t * C + c] = a[c];
      for (int32_t h0 = 0; h0 < n_l2; h0 += dk) {
        double ss = 0.0;
        for (int32_t i = 0; i < dk; ++i) ss += a[h0 + i] * a[h0 + i];
        double r = sqrt(ss + eps);
        for (int32_t i = 0; i < dk; ++i) y[t * C + h0 + i] = a[h0 + i] / r;
      }
      free(u);
      free(a);
    }
  }
  return OR_OK;
}

/* ---------------------------------------------------------------------------
 * The same convolution with a carried conv state (prime-rl page, "Summary":
 * causal_conv1d takes initial_state and output_final_state).  The state of
 * sequence n is the K-1 input rows just before its first token, oldest first:
 * cs_in[n][r][c] stands for x at position t0 - (K-1) + r (NULL: zeros, the
 * stateless convolution).  cs_out[n][r][c] is the input at position
 * t1 - (K-1) + r, taken from cs_in where that position precedes t0 (short
 * sequences), so that feeding it to the next call continues the sequence.
 * ------------------------------------------------------------------------- */

/* x at position p of sequence n (tokens [t0, t1)), reading the carried state
 * for positions before t0 */
static double x_or_state(int64_t p, int64_t t0, int32_t n, int32_t C, int32_t K, int32_t c,
                         const double* x, const double* cs_in) {
  if (p >= t0) return x[p * C + c];
  int64_t r = p - t0 + (K - 1);
  if (!cs_in || r < 0) return 0.0;
  return cs_in[((int64_t)n * (K - 1) + r) * C + c];
}

static void conv_silu_row_state(int64_t t, int64_t t0, int32_t n, int32_t C, int32_t K,
                                const double* x, const double* w, const double* cs_in, double* u,
                                double* a) {
  for (int32_t c = 0; c < C; ++c) {
    double acc = 0.0;
    for (int32_t j = 0; j < K; ++j)
      acc += w[(int64_t)c * K + j] * x_or_state(t - (K - 1) + j, t0, n, C, K, c, x, cs_in);
    u[c] = acc;
    a[c] = acc * sigm(acc);
  }
}

int oracle_conv_state_fwd(int64_t T, int32_t C, int32_t K, const double* x, const double* w,
                          const int32_t* cu, int32_t N, int32_t n_l2, int32_t dk, double eps,
                          const double* cs_in, double* y, double* cs_out) {
  if (T < 0 || C <= 0 || K <= 1 || N < 0 || n_l2 < 0 || n_l2 > C || (n_l2 && (dk <= 0 || n_l2 % dk)))
    return OR_ERR;
  for (int32_t n = 0; n < N; ++n) {
    int64_t t0 = cu[n], t1 = cu[n + 1];
#pragma omp parallel for schedule(static)
    for (int64_t t = t0; t < t1; ++t) {
      double* u = (double*)malloc(sizeof(double) * C);
      double* a = (double*)malloc(sizeof(double) * C);
      conv_silu_row_state(t, t0, n, C, K, x, w, cs_in, u, a);
      for (int32_t c = 0; c < C; ++c) y[t * C + c] = a[c];
      for (int32_t h0 = 0; h0 < n_l2; h0 += dk) {
        double ss = 0.0;
        for (int32_t i = 0; i < dk; ++i) ss += a[h0 + i] * a[h0 + i];
        double r = sqrt(ss + eps);
        for (int32_t i = 0; i < dk; ++i) y[t * C + h0 + i] = a[h0 + i] / r;
      }
      free(u);
      free(a);
    }
    if (cs_out)
      for (int32_t r = 0; r < K - 1; ++r)
        for (int32_t c = 0; c < C; ++c)
          cs_out[((int64_t)n * (K - 1) + r) * C + c] =
              x_or_state(t1 - (K - 1) + r, t0, n, C, K, c, x, cs_in);
  }
  return OR_OK;
}

/* Backward of oracle_conv_state_fwd: dy [T][C] and dcs_out [N][K-1][C] (NULL:
 * zero) -> dx [T][C], dw [C][K], dcs_in [N][K-1][C] (NULL: not wanted).
 * Input position p of sequence n feeds u at tokens p + (K-1) - j (tap j) of
 * the sequence, and the final state when p >= t1 - (K-1). */
int oracle_conv_state_bwd(int64_t T, int32_t C, int32_t K, const double* x, const double* w,
                          const int32_t* cu, int32_t N, int32_t n_l2, int32_t dk, double eps,
                          const double* cs_in, const double* dy, const double* dcs_out,
                          double* dx, double* dw, double* dcs_in) {
  if (T < 0 || C <= 0 || K <= 1 || N < 0 || n_l2 < 0 || n_l2 > C || (n_l2 && (dk <= 0 || n_l2 % dk)))
    return OR_ERR;
  double* du = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * C);
  for (int32_t n = 0; n < N; ++n) {
    int64_t t0 = cu[n], t1 = cu[n + 1];
#pragma omp parallel for schedule(static)
    for (int64_t t = t0; t < t1; ++t) {
      double* u = (double*)malloc(sizeof(double) * C);
      double* a = (double*)malloc(sizeof(double) * C);
      double* da = (double*)malloc(sizeof(double) * C);
      conv_silu_row_state(t, t0, n, C, K, x, w, cs_in, u, a);
      for (int32_t c = 0; c < C; ++c) da[c] = dy[t * C + c];
      /* L2 backward: y = a / r, r = sqrt(sum a^2 + eps)
       *   da = dy / r - a (a . dy) / r^3 */
      for (int32_t h0 = 0; h0 < n_l2; h0 += dk) {
        double ss = 0.0, ady = 0.0;
        for (int32_t i = 0; i < dk; ++i) {
          ss += a[h0 + i] * a[h0 + i];
          ady += a[h0 + i] * dy[t * C + h0 + i];
        }
        double r2 = ss + eps, r = sqrt(r2);
        for (int32_t i = 0; i < dk; ++i)
          da[h0 + i] = dy[t * C + h0 + i] / r - a[h0 + i] * ady / (r2 * r);
      }
      for (int32_t c = 0; c < C; ++c) {
        double sg = sigm(u[c]);
        du[t * C + c] = da[c] * sg * (1.0 + u[c] * (1.0 - sg));
      }
      free(u);
      free(a);
      free(da);
    }
  }
  /* gradient of input position p of sequence n (a token, or a state row) */
  for (int32_t n = 0; n < N; ++n) {
    int64_t t0 = cu[n], t1 = cu[n + 1];
#pragma omp parallel for schedule(static)
    for (int64_t p = t0 - (K - 1); p < t1; ++p) {
      for (int32_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < K; ++j) {
          int64_t t = p + (K - 1) - j;
          if (t >= t0 && t < t1) acc += w[(int64_t)c * K + j] * du[t * C + c];
        }
        int64_t rf = p - (t1 - (K - 1));   /* row of the final state holding p */
        if (dcs_out && rf >= 0) acc += dcs_out[((int64_t)n * (K - 1) + rf) * C + c];
        if (p >= t0) dx[p * C + c] = acc;
        else if (dcs_in) dcs_in[((int64_t)n * (K - 1) + (p - t0 + (K - 1))) * C + c] = acc;
      }
    }
  }
  /* dw[c][j] = sum over sequences, tokens t of du[t][c] x~[t-(K-1)+j][c] */
#pragma omp parallel for schedule(static)
  for (int32_t c = 0; c < C; ++c) {
    for (int32_t j = 0; j < K; ++j) {
      double acc = 0.0;
      for (int32_t n = 0; n < N; ++n) {
        int64_t t0 = cu[n], t1 = cu[n + 1];
        for (int64_t t = t0; t < t1; ++t)
          acc += du[t * C + c] * x_or_state(t - (K - 1) + j, t0, n, C, K, c, x, cs_in);
      }
      dw[(int64_t)c * K + j] = acc;
    }
  }
  free(du);
  return OR_OK;
}

/* Backward of oracle_conv_fwd.  dy: [T][C] -> dx: [T][C], dw: [C][K]. */
int oracle_conv_bwd(int64_t T, int32_t C, int32_t K, const double* x, const double* w,
                    const int32_t* cu, int32_t N, int32_t n_l2, int32_t dk, double eps,
                    const double* dy, double* dx, double* dw) {
  if (T < 0 || C <= 0 || K <= 0 || N < 0 || n_l2 < 0 || n_l2 > C || (n_l2 && (dk <= 0 || n_l2 % dk)))
    return OR_ERR;
  double* du = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * C);
  for (int32_t n = 0; n < N; ++n) {
    int64_t t0 = cu[n], t1 = cu[n + 1];
#pragma omp parallel for schedule(static)
    for (int64_t t = t0; t < t1; ++t) {
      double* u = (double*)malloc(sizeof(double) * C);
      double* a = (double*)malloc(sizeof(double) * C);
      double* da = (double*)malloc(sizeof(double) * C);
      conv_silu_row(t, t0, C, K, x, w, u, a);
      for (int32_t c = 0; c < C; ++c) da[c] = dy[t * C + c];
      /* L2 backward: y = a / r, r = sqrt(sum a^2 + eps)
       *   da = dy / r - a (a . dy) / r^3 */
      for (int32_t h0 = 0; h0 < n_l2; h0 += dk) {
        double ss = 0.0, ady = 0.0;
        for (int32_t i = 0; i < dk; ++i) {
          ss += a[h0 + i] * a[h0 + i];
          ady += a[h0 + i] * dy[t * C + h0 + i];
        }
        double r2 = ss + eps, r = sqrt(r2);
        for (int32_t i = 0; i < dk; ++i)
          da[h0 + i] = dy[t * C + h0 + i] / r - a[h0 + i] * ady / (r2 * r);
      }
      /* SiLU backward: d/du [u sigma(u)] = sigma(u) (1 + u (1 - sigma(u))) */
      for (int32_t c = 0; c < C; ++c) {
        double sg = sigm(u[c]);
        du[t * C + c] = da[c] * sg * (1.0 + u[c] * (1.0 - sg));
      }
      free(u);
      free(a);
      free(da);
    }
  }
  /* dx[s][c] = sum_j w[c][j] du[s+(K-1)-j][c] within the sequence of s */
  for (int32_t n = 0; n < N; ++n) {
    int64_t t0 = cu[n], t1 = cu[n + 1];
#pragma omp parallel for schedule(static)
    for (int64_t s = t0; s < t1; ++s) {
      for (int32_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < K; ++j) {
          int64_t t = s + (K - 1) - j;
          if (t < t1) acc += w[(int64_t)c * K + j] * du[t * C + c];
        }
        dx[s * C + c] = acc;
      }
    }
  }
  /* dw[c][j] = sum over sequences, tokens t of du[t][c] x[t-(K-1)+j][c] */
#pragma omp parallel for schedule(static)
  for (int32_t c = 0; c < C; ++c) {
    for (int32_t j = 0; j < K; ++j) {
      double acc = 0.0;
      for (int32_t n = 0; n < N; ++n) {
        int64_t t0 = cu[n], t1 = cu[n + 1];
        for (int64_t t = t0; t < t1; ++t) {
          int64_t s = t - (K - 1) + j;
          if (s >= t0) acc += du[t * C + c] * x[s * C + c];
        }
      }
      dw[(int64_t)c * K + j] = acc;
    }
  }
  free(du);
  return OR_OK;
}

/* ---------------------------------------------------------------------------
 * Gate: g = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h]);  beta = sigmoid(b).
 * a, b, g, beta: [T][H].
 * ------------------------------------------------------------------------- */
int oracle_gate_fwd(int64_t T, int32_t H, const double* a, const double* b, const double* A_log,
                    const double* dt_bias, double* g, double* beta) {
  if (T < 0 || H <= 0) return OR_ERR;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < H; ++h) {
      g[t * H + h] = -exp(A_log[h]) * softplus(a[t * H + h] + dt_bias[h]);
      beta[t * H + h] = sigm(b[t * H + h]);
    }
  return OR_OK;
}

int oracle_gate_bwd(int64_t T, int32_t H, const double* a, const double* b, const double* A_log,
                    const double* dt_bias, const double* dg, const double* dbeta, double* da,
                    double* db, double* dA_log, double* ddt_bias) {
  if (T < 0 || H <= 0) return OR_ERR;
  for (int32_t h = 0; h < H; ++h) {
    double sA = 0.0, sdt = 0.0;
    double A = exp(A_log[h]);
    for (int64_t t = 0; t < T; ++t) {
      double xin = a[t * H + h] + dt_bias[h];
      double g = -A * softplus(xin);
      /* d softplus / dx = sigmoid(x) */
      double dxin = dg[t * H + h] * (-A) * sigm(xin);
      da[t * H + h] = dxin;
      sdt += dxin;
      /* d g / d A_log = g (since g is linear in exp(A_log)) */
      sA += dg[t * H + h] * g;
      double bt = sigm(b[t * H + h]);
      db[t * H + h] = dbeta[t * H + h] * bt * (1.0 - bt);
    }
    dA_log[h] = sA;
    ddt_bias[h] = sdt;
  }
  return OR_OK;
}

/* ---------------------------------------------------------------------------
 * Gated delta rule, token by token.
 *
 * q, k: [T][Hk][dk]; v, o: [T][Hv][dv]; g, beta: [T][Hv];
 * S0, S_final: [N][Hv][dv][dk] (S0 may be NULL = zero, S_final may be NULL).
 * Value head h uses key head h / (Hv / Hk).
 * ------------------------------------------------------------------------- */
static int delta_args_ok(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv) {
  return T >= 0 && N >= 0 && Hk > 0 && Hv > 0 && Hv % Hk == 0 && dk > 0 && dv > 0;
}

/* One token of the recurrence on S (dv x dk, row-major), in the order
 *   S <- alpha S;  p = S k;  delta = beta (v - p);  S <- S + delta k^T.
 * Writes p and delta if given. */
static void delta_step(double* S, int32_t dv, int32_t dk, double alpha, double beta,
                       const double* kt, const double* vt, double* p, double* delta) {
  for (int32_t i = 0; i < dv * dk; ++i) S[i] *= alpha;
  for (int32_t i = 0; i < dv; ++i) {
    double acc = 0.0;
    for (int32_t j = 0; j < dk; ++j) acc += S[i * dk + j] * kt[j];
    double di = beta * (vt[i] - acc);
    if (p) p[i] = acc;
    if (delta) delta[i] = di;
    for (int32_t j = 0; j < dk; ++j) S[i * dk + j] += di * kt[j];
  }
}

int oracle_delta_fwd(int64_t T, int32_t N, const int32_t* cu, int32_t Hk, int32_t Hv, int32_t dk,
                     int32_t dv, const double* q, const double* k, const double* v,
                     const double* g, const double* beta, double scale, const double* S0,
                     double* o, double* S_final) {
  if (!delta_args_ok(T, N, Hk, Hv, dk, dv)) return OR_ERR;
  int32_t G = Hv / Hk;
  int64_t SS = (int64_t)dv * dk;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < Hv; ++h) {
      int32_t kh = h / G;
      double* S = (double*)malloc(sizeof(double) * SS);
      if (S0) memcpy(S, S0 + ((int64_t)n * Hv + h) * SS, sizeof(double) * SS);
      else memset(S, 0, sizeof(double) * SS);
      for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
        const double* kt = k + (t * Hk + kh) * dk;
        const double* qt = q + (t * Hk + kh) * dk;
        const double* vt = v + (t * Hv + h) * dv;
        delta_step(S, dv, dk, exp(g[t * Hv + h]), beta[t * Hv + h], kt, vt, NULL, NULL);
        double* ot = o + (t * Hv + h) * dv;
        for (int32_t i = 0; i < dv; ++i) {
          double acc = 0.0;
          for (int32_t j = 0; j < dk; ++j) acc += S[i * dk + j] * (scale * qt[j]);
          ot[i] = acc;
        }
      }
      if (S_final) memcpy(S_final + ((int64_t)n * Hv + h) * SS, S, sizeof(double) * SS);
      free(S);
    }
  }
  return OR_OK;
}

/* Backward of oracle_delta_fwd by backpropagation through time.  States are
 * checkpointed every `seg` tokens and recomputed segment by segment in
 * reverse.  dq and dk sum over the value heads of a group in ascending h.
 * dS_final may be NULL (zero); dS0 may be NULL (not wanted). */
int oracle_delta_bwd(int64_t T, int32_t N, const int32_t* cu, int32_t Hk, int32_t Hv, int32_t dk,
                     int32_t dv, const double* q, const double* k, const double* v,
                     const double* g, const double* beta, double scale, const double* S0,
                     const double* dout, const double* dS_final, double* dq, double* dkk,
                     double* dvv, double* dg, double* dbeta, double* dS0) {
  if (!delta_args_ok(T, N, Hk, Hv, dk, dv)) return OR_ERR;
  const int32_t seg = 64;
  int32_t G = Hv / Hk;
  int64_t SS = (int64_t)dv * dk;
  memset(dq, 0, sizeof(double) * (size_t)T * Hk * dk);
  memset(dkk, 0, sizeof(double) * (size_t)T * Hk * dk);
  /* parallel over (sequence, key head): a key head's value heads run in
   * ascending order inside one thread, so dq/dk sums are ordered. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t n = 0; n < N; ++n) {
    for (int32_t kh = 0; kh < Hk; ++kh) {
      int64_t t0 = cu[n], t1 = cu[n + 1], L = t1 - t0;
      int64_t nseg = (L + seg - 1) / seg;
      double* ckpt = (double*)malloc(sizeof(double) * SS * (size_t)(nseg > 0 ? nseg : 1));
      double* Sseg = (double*)malloc(sizeof(double) * SS * (seg + 1));
      double* dS = (double*)malloc(sizeof(double) * SS);
      double* dSt = (double*)malloc(sizeof(double) * SS);
      double* p = (double*)malloc(sizeof(double) * dv);
      double* dl = (double*)malloc(sizeof(double) * dv);
      double* ddl = (double*)malloc(sizeof(double) * dv);
      double* dp = (double*)malloc(sizeof(double) * dv);
      for (int32_t hh = 0; hh < G; ++hh) {
        int32_t h = kh * G + hh;
        /* forward: checkpoint the state entering every segment */
        double* S = Sseg;
        if (S0) memcpy(S, S0 + ((int64_t)n * Hv + h) * SS, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (int64_t sgi = 0; sgi < nseg; ++sgi) {
          memcpy(ckpt + sgi * SS, S, sizeof(double) * SS);
          int64_t a0 = t0 + sgi * seg, a1 = a0 + seg < t1 ? a0 + seg : t1;
          for (int64_t t = a0; t < a1; ++t)
            delta_step(S, dv, dk, exp(g[t * Hv + h]), beta[t * Hv + h], k + (t * Hk + kh) * dk,
                       v + (t * Hv + h) * dv, NULL, NULL);
        }
        /* reverse */
        if (dS_final) memcpy(dS, dS_final + ((int64_t)n * Hv + h) * SS, sizeof(double) * SS);
        else memset(dS, 0, sizeof(double) * SS);
        for (int64_t sgi = nseg - 1; sgi >= 0; --sgi) {
          int64_t a0 = t0 + sgi * seg, a1 = a0 + seg < t1 ? a0 + seg : t1;
          /* Sseg[i] = state entering token a0+i (i.e. after token a0+i-1) */
          memcpy(Sseg, ckpt + sgi * SS, sizeof(double) * SS);
          for (int64_t t = a0; t < a1; ++t) {
            double* Sn = Sseg + (t - a0 + 1) * SS;
            memcpy(Sn, Sseg + (t - a0) * SS, sizeof(double) * SS);
            delta_step(Sn, dv, dk, exp(g[t * Hv + h]), beta[t * Hv + h], k + (t * Hk + kh) * dk,
                       v + (t * Hv + h) * dv, NULL, NULL);
          }
          for (int64_t t = a1 - 1; t >= a0; --t) {
            const double* Sp = Sseg + (t - a0) * SS;      /* S_{t-1} */
            const double* St = Sseg + (t - a0 + 1) * SS;  /* S_t */
            const double* kt = k + (t * Hk + kh) * dk;
            const double* qt = q + (t * Hk + kh) * dk;
            const double* vt = v + (t * Hv + h) * dv;
            const double* dot = dout + (t * Hv + h) * dv;
            double alpha = exp(g[t * Hv + h]), bt = beta[t * Hv + h];
            double* dqt = dq + (t * Hk + kh) * dk;
            double* dkt = dkk + (t * Hk + kh) * dk;
            /* o = S_t (scale q):  dS += do (scale q)^T;  dq += scale S_t^T do */
            for (int32_t i = 0; i < dv; ++i)
              for (int32_t j = 0; j < dk; ++j) dS[i * dk + j] += dot[i] * scale * qt[j];
            for (int32_t j = 0; j < dk; ++j) {
              double acc = 0.0;
              for (int32_t i = 0; i < dv; ++i) acc += St[i * dk + j] * dot[i];
              dqt[j] += scale * acc;
            }
            /* recompute p = (alpha S_{t-1}) k and delta = beta (v - p) */
            for (int32_t i = 0; i < dv; ++i) {
              double acc = 0.0;
              for (int32_t j = 0; j < dk; ++j) acc += alpha * Sp[i * dk + j] * kt[j];
              p[i] = acc;
              dl[i] = bt * (vt[i] - acc);
            }
            /* S_t = St~ + delta k^T:  d delta = dS k;  dk += dS^T delta */
            for (int32_t i = 0; i < dv; ++i) {
              double acc = 0.0;
              for (int32_t j = 0; j < dk; ++j) acc += dS[i * dk + j] * kt[j];
              ddl[i] = acc;
            }
            for (int32_t j = 0; j < dk; ++j) {
              double acc = 0.0;
              for (int32_t i = 0; i < dv; ++i) acc += dS[i * dk + j] * dl[i];
              dkt[j] += acc;
            }
            /* delta = beta (v - p) */
            double dbt = 0.0;
            for (int32_t i = 0; i < dv; ++i) {
              dbt += ddl[i] * (vt[i] - p[i]);
              dvv[(t * Hv + h) * dv + i] = bt * ddl[i];
              dp[i] = -bt * ddl[i];
            }
            dbeta[t * Hv + h] = dbt;
            /* p = St~ k with St~ = alpha S_{t-1}:
             *   dSt~ = dS + dp k^T;  dk += St~^T dp */
            for (int32_t j = 0; j < dk; ++j) {
              double acc = 0.0;
              for (int32_t i = 0; i < dv; ++i) acc += alpha * Sp[i * dk + j] * dp[i];
              dkt[j] += acc;
            }
            for (int32_t i = 0; i < dv; ++i)
              for (int32_t j = 0; j < dk; ++j) dSt[i * dk + j] = dS[i * dk + j] + dp[i] * kt[j];
            /* St~ = exp(g) S_{t-1}: dg = <dSt~, St~>;  dS_{t-1} = alpha dSt~ */
            double dgt = 0.0;
            for (int32_t i = 0; i < dv * dk; ++i) dgt += dSt[i] * alpha * Sp[i];
            dg[t * Hv + h] = dgt;
            for (int32_t i = 0; i < dv * dk; ++i) dS[i] = alpha * dSt[i];
          }
        }
        if (dS0) memcpy(dS0 + ((int64_t)n * Hv + h) * SS, dS, sizeof(double) * SS);
      }
      free(ckpt);
      free(Sseg);
      free(dS);
      free(dSt);
      free(p);
      free(dl);
      free(ddl);
      free(dp);
    }
  }
  return OR_OK;
}

/* ---------------------------------------------------------------------------
 * Gated zero-centred RMSNorm over rows of length d:
 *   n = o / sqrt(mean(o^2) + eps);  y = n * (1 + w) * act(z)
 * act = 0: SiLU  z sigma(z);  act = 1: sigmoid  sigma(z).
 * ------------------------------------------------------------------------- */
static double act_f(int act, double z) { return act == 0 ? z * sigm(z) : sigm(z); }
static double act_df(int act, double z) {
  double s = sigm(z);
  return act == 0 ? s * (1.0 + z * (1.0 - s)) : s * (1.0 - s);
}

int oracle_norm_fwd(int64_t rows, int32_t d, const double* o, const double* z, const double* w,
                    double eps, int act, double* y) {
  if (rows < 0 || d <= 0 || (act != 0 && act != 1)) return OR_ERR;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) ss += o[r * d + i] * o[r * d + i];
    double rho = 1.0 / sqrt(ss / d + eps);
    for (int32_t i = 0; i < d; ++i)
      y[r * d + i] = o[r * d + i] * rho * (1.0 + w[i]) * act_f(act, z[r * d + i]);
  }
  return OR_OK;
}

int oracle_norm_bwd(int64_t rows, int32_t d, const double* o, const double* z, const double* w,
                    double eps, int act, const double* dy, double* dout, double* dz, double* dw) {
  if (rows < 0 || d <= 0 || (act != 0 && act != 1)) return OR_ERR;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) ss += o[r * d + i] * o[r * d + i];
    double rho = 1.0 / sqrt(ss / d + eps);
    /* dn = dy (1 + w) act(z);  do = rho (dn - n mean(dn n)) */
    double m = 0.0;
    for (int32_t i = 0; i < d; ++i) {
      double n = o[r * d + i] * rho;
      double dn = dy[r * d + i] * (1.0 + w[i]) * act_f(act, z[r * d + i]);
      m += dn * n;
    }
    m /= d;
    for (int32_t i = 0; i < d; ++i) {
      double n = o[r * d + i] * rho;
      double dn = dy[r * d + i] * (1.0 + w[i]) * act_f(act, z[r * d + i]);
      dout[r * d + i] = rho * (dn - n * m);
      dz[r * d + i] = dy[r * d + i] * n * (1.0 + w[i]) * act_df(act, z[r * d + i]);
    }
  }
  /* dw[i] = sum over rows (in row order) of dy n act(z) */
  for (int32_t i = 0; i < d; ++i) dw[i] = 0.0;
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) ss += o[r * d + i] * o[r * d + i];
    double rho = 1.0 / sqrt(ss / d + eps);
    for (int32_t i = 0; i < d; ++i)
      dw[i] += dy[r * d + i] * o[r * d + i] * rho * act_f(act, z[r * d + i]);
  }
  return OR_OK;
}
