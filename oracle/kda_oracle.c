/*
 * KDA recurrent prefill forward -- CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * This file is the plain, slow, fp64 reference that the HIP path is checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no source with the GPU library and includes
 * none of its headers.
 *
 * What it computes (per sequence n, head h; state S is V x K, stored [N,H,V,K]):
 *
 *   gate      lam_t[k] = lb * sigmoid(exp(A_log[h]) * (g_t[k] + dt_bias[h,k]))
 *             (natural-log decay; the pages fix the inputs g, A_log, dt_bias,
 *             lower_bound and the per-token range [lb, 0] -- FlashInfer PR #4262
 *             summary, section 2 "Chunk-32 Through Fixed-Anchor Exponent
 *             Centering" and section 12 "Strict Dispatch and Safe Fallback";
 *             the formula itself is a reading: parity unpinned against any
 *             printed gate values, since no page prints one; its closed-form
 *             values, limits and range are pinned by the test suite)
 *   norms     qh_t = q_t / sqrt(|q_t|^2 + eps),  kh_t = k_t / sqrt(|k_t|^2 + eps)
 *             (in-kernel Q/K L2 normalisation, section 12 of the same page)
 *   beta      b_t = sigmoid(beta_t)   (the beta input is a logit, section 12)
 *   decay     S <- S * diag(exp(lam_t))                 (decay first ...)
 *   delta     S <- S + b_t (v_t - S kh_t) kh_t^T         (... then the update)
 *   output    o_t = scale * S qh_t                      (read after the update)
 *
 * The decay-before-update and read-after-update order are the ones the page's
 * chunk decomposition fixes (section 3 "Intra-Chunk and Inter-Chunk
 * Decomposition": S_d = S_old diag(a) with an inclusive prefix, and a lower
 * triangular Mqk that keeps its diagonal).  The state starts from
 * initial_state[n] (zeros when absent) and nothing carries between sequences
 * ("How FlashKDA Manages Recurrent State Across Sequences and Batch Modes",
 * variable-length mode).  Batched mode is the same computation with
 * cu_seqlens = [0, T, 2T, ...] over the flattened [B*T] token axis.
 *
 * Everything is fp64 and strictly token by token: no chunking, no blocking,
 * no reordering of the sums beyond the plain loops below.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_EPS 1e-6

static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Per-token natural-log decay of one token row: lam[k] for k < K. */
static void oracle_gate_row(const double* g_row, const double* dt_bias_h, double a_coef,
                            double lower_bound, int64_t K, double* lam) {
  for (int64_t k = 0; k < K; ++k)
    lam[k] = lower_bound * oracle_sigmoid(a_coef * (g_row[k] + dt_bias_h[k]));
}

/* 1 / sqrt(sum x^2 + eps) of one row. */
static double oracle_inv_norm(const double* x, int64_t K) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k) s += x[k] * x[k];
  return 1.0 / sqrt(s + KDA_ORACLE_EPS);
}

/*
 * Exported: the gate on its own, lam[T,H,K] from g[T,H,K], so the tests can pin
 * its closed-form values and its range without running the recurrence.
 */
void kda_oracle_gate(const double* g, const double* A_log, const double* dt_bias,
                     double lower_bound, int64_t T, int64_t H, int64_t K, double* lam) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < H; ++h)
      oracle_gate_row(g + (t * H + h) * K, dt_bias + h * K, exp(A_log[h]), lower_bound, K,
                      lam + (t * H + h) * K);
}

/*
 * Exported: the forward pass.
 *   q, k, g   [T_total, H, K]        (fp64, the exact values of the bf16 inputs)
 *   v         [T_total, H, V]
 *   beta      [T_total, H]           (logits)
 *   A_log     [H], dt_bias [H, K]
 *   initial_state [N, H, V, K] or NULL (zeros)
 *   cu_seqlens [N+1] host array: sequence n covers tokens [cu[n], cu[n+1])
 *   out       [T_total, H, V]        written for every token of every sequence
 *   final_state [N, H, V, K]         written (NULL: not written)
 *   nthreads  OpenMP threads (<= 0: the runtime default)
 * Returns 0, or -1 if cu_seqlens is not a non-decreasing partition of
 * [0, T_total] (nothing is written then).
 */
int kda_oracle_fwd(const double* q, const double* k, const double* v, const double* g,
                   const double* beta, double scale, const double* A_log,
                   const double* dt_bias, double lower_bound, const double* initial_state,
                   double* out, double* final_state, const int64_t* cu_seqlens, int64_t N,
                   int64_t T_total, int64_t H, int64_t K, int64_t V, int nthreads) {
  if (N < 0 || cu_seqlens[0] != 0 || cu_seqlens[N] != T_total) return -1;
  for (int64_t n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

  const int64_t units = N * H;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int64_t n = u / H, h = u % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)(V * K));
    double* lam = (double*)malloc(sizeof(double) * (size_t)K);
    double* alpha = (double*)malloc(sizeof(double) * (size_t)K);
    double* kh = (double*)malloc(sizeof(double) * (size_t)K);
    double* qh = (double*)malloc(sizeof(double) * (size_t)K);
    const double a_coef = exp(A_log[h]);

    const double* S0 = initial_state ? initial_state + (n * H + h) * V * K : NULL;
    for (int64_t i = 0; i < V * K; ++i) S[i] = S0 ? S0[i] : 0.0;

    for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
      const int64_t row = t * H + h;
      oracle_gate_row(g + row * K, dt_bias + h * K, a_coef, lower_bound, K, lam);
      const double rq = oracle_inv_norm(q + row * K, K);
      const double rk = oracle_inv_norm(k + row * K, K);
      for (int64_t j = 0; j < K; ++j) {
        qh[j] = q[row * K + j] * rq;
        kh[j] = k[row * K + j] * rk;
        alpha[j] = exp(lam[j]);
      }
      const double b = oracle_sigmoid(beta[row]);

      /* decay: S <- S diag(exp(lam)) */
      for (int64_t i = 0; i < V; ++i)
        for (int64_t j = 0; j < K; ++j) S[i * K + j] *= alpha[j];

      /* delta rule: S <- S + b (v - S kh) kh^T */
      for (int64_t i = 0; i < V; ++i) {
        double pred = 0.0;
        for (int64_t j = 0; j < K; ++j) pred += S[i * K + j] * kh[j];
        const double d = b * (v[row * V + i] - pred);
        for (int64_t j = 0; j < K; ++j) S[i * K + j] += d * kh[j];
      }

      /* output after the update: o = scale * S qh */
      for (int64_t i = 0; i < V; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < K; ++j) acc += S[i * K + j] * qh[j];
        out[row * V + i] = scale * acc;
      }
    }

    if (final_state) {
      double* SF = final_state + (n * H + h) * V * K;
      for (int64_t i = 0; i < V * K; ++i) SF[i] = S[i];
    }
    free(S);
    free(lam);
    free(alpha);
    free(kh);
    free(qh);
  }
  return 0;
}
