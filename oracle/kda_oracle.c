/*
 * KDA oracle, C twin of oracle/kda_ref.py for workloads too large for numpy
 * loops.  TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and
 * the benchmark's CPU-baseline leg; never by the GPU library, with which it
 * shares no code.
 *
 * Plain fp64, token by token, one (batch, head) per OpenMP task.  Follows the
 * recurrence of "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
 * (hs-black.github.io/posts/kimi-k3), section 2.1:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 * applied in the equivalent rank-1 order
 *     S <- Diag(alpha_t) S;  S <- S + beta_t k_t (v_t - S^T k_t)^T,
 * with alpha_t = exp(g_min * sigmoid(exp(A_h) z_t)) (section 2.2; decay == 0)
 * or, for the Kimi Linear map that section 2.2 compares it with (decay == 1),
 * alpha_t = exp(-exp(A_h) softplus(z_t)), and the gate
 * y_t = sigmoid(gate_t) * RMSNorm(o_t) (section 2.3).
 * q and k are L2-normalised first when l2norm != 0: x / sqrt(sum x^2 + eps).
 *
 * Layouts: q, k, z [B, T, H, dk]; v, gate [B, T, H, dv]; beta [B, T, H];
 * A [H]; w [H, dv] or NULL; S0 and S_T [B, H, dk, dv] (row = key channel);
 * o and y [B, T, H, dv].  All inputs fp32 (bf16 values widen exactly),
 * all outputs fp64.  Any output pointer may be NULL.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double sigmoid_stable(double x) {
  if (x >= 0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

/* softplus(x) = log(1 + e^x) without overflow */
static double softplus_stable(double x) { return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x))); }

int kda_oracle_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                       const float* q, const float* k, const float* v, const float* beta,
                       const float* z, const float* A, double g_min, double scale, int l2norm,
                       double l2_eps, const double* S0, const float* gate, const float* w,
                       double rms_eps, double* o, double* y, double* S_T, int nthreads, int decay) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (!q || !k || !v || !beta || !z || !A) return -1;
  if (decay != 0 && decay != 1) return -1;
  if (y && !gate) return -1;
  const int64_t tasks = B * H;
  int fail = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
  for (int64_t task = 0; task < tasks; ++task) {
    const int64_t b = task / H, h = task % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
    double* qv = (double*)malloc(sizeof(double) * (size_t)dk);
    double* kv = (double*)malloc(sizeof(double) * (size_t)dk);
    double* al = (double*)malloc(sizeof(double) * (size_t)dk);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* ot = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !qv || !kv || !al || !u || !ot) {
      fail = 1;
    } else {
      if (S0)
        memcpy(S, S0 + (b * H + h) * dk * dv, sizeof(double) * (size_t)(dk * dv));
      else
        memset(S, 0, sizeof(double) * (size_t)(dk * dv));
      const double eA = exp((double)A[h]);
      for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        const float* qr = q + row * dk;
        const float* kr = k + row * dk;
        const float* zr = z + row * dk;
        const float* vr = v + row * dv;
        const double bt = (double)beta[row];
        double sq = 0.0, sk = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          qv[i] = (double)qr[i];
          kv[i] = (double)kr[i];
          sq += qv[i] * qv[i];
          sk += kv[i] * kv[i];
        }
        const double rq = l2norm ? 1.0 / sqrt(sq + l2_eps) : 1.0;
        const double rk = l2norm ? 1.0 / sqrt(sk + l2_eps) : 1.0;
        for (int64_t i = 0; i < dk; ++i) {
          qv[i] *= rq * scale;
          kv[i] *= rk;
          al[i] = decay == 0 ? exp(g_min * sigmoid_stable(eA * (double)zr[i]))
                             : exp(-eA * softplus_stable((double)zr[i]));
        }
        /* S <- Diag(alpha) S */
        for (int64_t i = 0; i < dk; ++i) {
          double* Si = S + i * dv;
          for (int64_t j = 0; j < dv; ++j) Si[j] *= al[i];
        }
        /* u = beta (v - S^T k) */
        for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          const double* Si = S + i * dv;
          for (int64_t j = 0; j < dv; ++j) u[j] += Si[j] * kv[i];
        }
        for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vr[j] - u[j]);
        /* S <- S + k u^T ; o = S^T q */
        for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          double* Si = S + i * dv;
          for (int64_t j = 0; j < dv; ++j) {
            Si[j] += kv[i] * u[j];
            ot[j] += Si[j] * qv[i];
          }
        }
        if (o) memcpy(o + row * dv, ot, sizeof(double) * (size_t)dv);
        if (y) {
          double ms = 0.0;
          for (int64_t j = 0; j < dv; ++j) ms += ot[j] * ot[j];
          const double rr = 1.0 / sqrt(ms / (double)dv + rms_eps);
          const float* gr = gate + row * dv;
          for (int64_t j = 0; j < dv; ++j) {
            const double wj = w ? (double)w[h * dv + j] : 1.0;
            y[row * dv + j] = sigmoid_stable((double)gr[j]) * ot[j] * rr * wj;
          }
        }
      }
      if (S_T) memcpy(S_T + (b * H + h) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
    }
    free(S);
    free(qv);
    free(kv);
    free(al);
    free(u);
    free(ot);
  }
  return fail ? -2 : 0;
}
