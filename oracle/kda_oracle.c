/*
 * Plain fp64 CPU oracle of the KDA (Kimi Delta Attention) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this code.  It shares nothing with the
 * GPU library: no headers, no helpers, no constants.
 *
 * What it computes, token by token, for every sequence n and head h
 * (per-channel gated delta rule):
 *
 *   q^_t = q_t / sqrt(sum q_t^2 + eps),  k^_t = k_t / sqrt(sum k_t^2 + eps)
 *   beta_t = sigmoid(raw_beta_t)
 *   g_{t,c} = lower_bound * sigmoid(exp(A_log[h]) * (raw_gate_{t,c} + dt_bias[h,c]))
 *   S <- Diag(exp(g_t)) S                       (decay every row of the K x V state)
 *   delta = beta_t * (v_t - S^T k^_t)           (delta-rule error)
 *   S <- S + k^_t delta^T                       (write)
 *   o_t = scale * S^T q^_t                      (read the updated state)
 *
 * Sources: the in-kernel flags of the fla chunk_kda call on the instagit
 * FlashKDA page ("Usage Examples": use_qk_l2norm_in_kernel,
 * use_beta_sigmoid_in_kernel, use_gate_in_kernel with A_log, dt_bias,
 * lower_bound, safe_gate) and the argument roles of the 14-argument
 * torch.ops._flashkda_C.fwd call in the vLLM PR report ("关键源码片段").  The
 * pages do not print the recurrence or the gate formula; the gate formula
 * above is the explicit reading this project adopts, and the update order
 * (decay, then erase/write, output from the updated state) is the standard
 * gated delta rule S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,
 * o_t = scale S_t^T q_t.  eps = 1e-6 is also a reading (the pages are silent).
 *
 * Inputs arrive as raw bf16 bit patterns (uint16) and are widened exactly.
 *
 * Variants (the chunk_kda flags on the same page, each switching one in-kernel
 * step off), selected by the bits of `flags`:
 *   ORACLE_GATE_GIVEN  raw_gate already holds g (natural-log decay), which must
 *                      lie in [lower_bound, 0]: the range the in-kernel gate
 *                      maps into, read as the bound that safe_gate=True with
 *                      lower_bound puts on the decay.  A value outside it is
 *                      not an input of the method; the call is rejected (-2).
 *                      A_log, dt_bias unused
 *   ORACLE_BETA_GIVEN  raw_beta already holds beta (no sigmoid)
 *   ORACLE_NO_QK_NORM  q^ = q, k^ = k (no L2 normalisation)
 *   ORACLE_STATE_VK    initial/final states stored transposed, [N, H, V, K]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_L2_EPS 1e-6
#define ORACLE_GATE_GIVEN 1
#define ORACLE_BETA_GIVEN 2
#define ORACLE_NO_QK_NORM 4
#define ORACLE_STATE_VK 8

static double widen_bf16(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* out[c] = x[c] / sqrt(sum_c x[c]^2 + eps), or x[c] unchanged if !normalise */
static void l2_normalise(const uint16_t* x, int64_t n, double* out, int normalise) {
  double ss = 0.0;
  for (int64_t c = 0; c < n; ++c) {
    double xc = widen_bf16(x[c]);
    out[c] = xc;
    ss += xc * xc;
  }
  if (!normalise) return;
  double r = 1.0 / sqrt(ss + ORACLE_L2_EPS);
  for (int64_t c = 0; c < n; ++c) out[c] *= r;
}

int kda_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * q, k, raw_gate: bf16 bits [T_total, H, K]; v: [T_total, H, V]; raw_beta: [T_total, H]
 * A_log fp32 [H]; dt_bias fp32 [H, K]; initial_state fp32 [N, H, K, V] or NULL (zeros)
 * cu_seqlens int32 [N+1] (host); heads: the n_heads head indices to evaluate.
 * out: fp64 [T_total, n_heads, V]; final_state: fp64 [N, n_heads, K, V] (may be NULL).
 * n_threads <= 0 keeps the OpenMP default; flags: ORACLE_* bits above.
 * Returns 0, -1 on bad sizes, or -2 for a given gate outside [lower_bound, 0].
 */
int kda_oracle_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* raw_gate, const uint16_t* raw_beta, double scale,
                   const float* A_log, const float* dt_bias, double lower_bound,
                   const float* initial_state, const int32_t* cu_seqlens, int64_t N,
                   int64_t T_total, int64_t H, int64_t K, int64_t V, const int32_t* heads,
                   int64_t n_heads, double* out, double* final_state, int n_threads, int flags) {
  if (N < 1 || H < 1 || K < 1 || V < 1 || n_heads < 1) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_total) return -1;
  for (int64_t n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  for (int64_t i = 0; i < n_heads; ++i)
    if (heads[i] < 0 || heads[i] >= H) return -1;
  if (flags & ORACLE_GATE_GIVEN)
    for (int64_t i = 0; i < T_total * H * K; ++i) {
      const double g = widen_bf16(raw_gate[i]);
      if (!(g >= lower_bound && g <= 0.0)) return -2;
    }
#ifdef _OPENMP
  /* the thread count applies to this call only (no process-wide OpenMP setting) */
  const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#else
  (void)n_threads;
#endif

  int64_t jobs = N * n_heads;
#pragma omp parallel num_threads(nt)
  {
    double* S = (double*)malloc(sizeof(double) * K * V);
    double* qh = (double*)malloc(sizeof(double) * K);
    double* kh = (double*)malloc(sizeof(double) * K);
    double* alpha = (double*)malloc(sizeof(double) * K);
    double* delta = (double*)malloc(sizeof(double) * V);
    double* acc = (double*)malloc(sizeof(double) * V);
#pragma omp for schedule(dynamic, 1)
    for (int64_t job = 0; job < jobs; ++job) {
      int64_t n = job / n_heads, hi = job % n_heads, h = heads[hi];
      /* initial state: S[c][j] at c*V + j, or at j*K + c in the transposed layout */
      const int vk = (flags & ORACLE_STATE_VK) != 0;
      for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j)
          S[c * V + j] = initial_state
                             ? (double)initial_state[(n * H + h) * K * V + (vk ? j * K + c : c * V + j)]
                             : 0.0;
      double gate_mul = (flags & ORACLE_GATE_GIVEN) ? 0.0 : exp((double)A_log[h]);
      for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
        int64_t th = t * H + h;
        int normalise = (flags & ORACLE_NO_QK_NORM) == 0;
        l2_normalise(q + th * K, K, qh, normalise);
        l2_normalise(k + th * K, K, kh, normalise);
        double rb = widen_bf16(raw_beta[th]);
        double beta = (flags & ORACLE_BETA_GIVEN) ? rb : sigmoid(rb);
        for (int64_t c = 0; c < K; ++c) {
          double rg = widen_bf16(raw_gate[th * K + c]);
          double g;
          if (flags & ORACLE_GATE_GIVEN)
            g = rg; /* checked above to lie in [lower_bound, 0] */
          else
            g = lower_bound * sigmoid(gate_mul * (rg + (double)dt_bias[h * K + c]));
          alpha[c] = exp(g);
        }
        /* decay: S <- Diag(alpha) S */
        for (int64_t c = 0; c < K; ++c)
          for (int64_t j = 0; j < V; ++j) S[c * V + j] *= alpha[c];
        /* prediction S^T k^ and delta = beta (v - S^T k^) */
        for (int64_t j = 0; j < V; ++j) acc[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
          for (int64_t j = 0; j < V; ++j) acc[j] += S[c * V + j] * kh[c];
        for (int64_t j = 0; j < V; ++j) delta[j] = beta * (widen_bf16(v[th * V + j]) - acc[j]);
        /* write: S <- S + k^ delta^T */
        for (int64_t c = 0; c < K; ++c)
          for (int64_t j = 0; j < V; ++j) S[c * V + j] += kh[c] * delta[j];
        /* output: o = scale S^T q^ */
        for (int64_t j = 0; j < V; ++j) acc[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
          for (int64_t j = 0; j < V; ++j) acc[j] += S[c * V + j] * qh[c];
        for (int64_t j = 0; j < V; ++j) out[(t * n_heads + hi) * V + j] = scale * acc[j];
      }
      if (final_state)
        for (int64_t c = 0; c < K; ++c)
          for (int64_t j = 0; j < V; ++j)
            final_state[(n * n_heads + hi) * K * V + (vk ? j * K + c : c * V + j)] = S[c * V + j];
    }
    free(S); free(qh); free(kh); free(alpha); free(delta); free(acc);
  }
  return 0;
}
