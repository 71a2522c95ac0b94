/*
 * Plain fp64 CPU oracle for the generalized linear-attention recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP path is checked against; it shares no code with that path.  Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark load it.
 *
 * Every routine here follows the plain definition, token by token, forming
 * the d_k x d_k transition matrix P_t explicitly:
 *
 *   S_t = P_t S_{t-1} + K_t V_t^T,        o_t = S_t^T q_t
 *
 * (HDLA note, "Key design 3": the general recurrence with decay
 * P_t = D_t - A_t B_t^T of rank r_ab and a write K_t V_t^T of rank r_kv.)
 * The chunk-wise method reaches this result exactly up to rounding (HLA note,
 * "Affine maps and closure under composition": chunk summaries carry no
 * approximation error), so the oracle is the definition, not the algorithm.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q    [BH, T, dk]          K [BH, T, r_kv, dk]     V [BH, T, r_kv, dv]
 *   ld   [BH, T, dk]  (per-channel log-decay, D_t = diag(exp(ld_t)))
 *        [BH, T]      (scalar log-decay, D_t = exp(ld_t) I)
 *   A, B [BH, T, r_ab, dk]    S0, Sfin [BH, dk, dv]   out [BH, T, dv]
 * Independent (batch, head) rows are spread over OpenMP threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_ENOMEM -1
#define ORACLE_EINVAL -2

static int set_threads(int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

/* S <- P S, P is n x n, S is n x m; tmp has n*m doubles. */
static void apply_left(int n, int m, const double* P, double* S, double* tmp) {
  for (int i = 0; i < n; ++i) {
    double* row = tmp + (size_t)i * m;
    for (int c = 0; c < m; ++c) row[c] = 0.0;
    for (int j = 0; j < n; ++j) {
      const double p = P[(size_t)i * n + j];
      if (p == 0.0) continue;
      const double* srow = S + (size_t)j * m;
      for (int c = 0; c < m; ++c) row[c] += p * srow[c];
    }
  }
  memcpy(S, tmp, sizeof(double) * (size_t)n * m);
}

/* out_t = S^T q : out[c] = sum_i S[i][c] q[i]. */
static void readout(int dk, int dv, const double* S, const double* q, double* out) {
  for (int c = 0; c < dv; ++c) out[c] = 0.0;
  for (int i = 0; i < dk; ++i) {
    const double qi = q[i];
    const double* srow = S + (size_t)i * dv;
    for (int c = 0; c < dv; ++c) out[c] += srow[c] * qi;
  }
}

/* P = diag(exp(ld)) - sum_r A_r B_r^T  (HDLA note, "Key design 3": D_t - A_t B_t^T). */
static void form_generic_P(int dk, int r_ab, int scalar_decay, const double* ld,
                           const double* A, const double* B, double* P) {
  for (int i = 0; i < dk; ++i) {
    for (int j = 0; j < dk; ++j) {
      double p = 0.0;
      if (i == j) p = exp(scalar_decay ? ld[0] : ld[i]);
      for (int r = 0; r < r_ab; ++r) p -= A[(size_t)r * dk + i] * B[(size_t)r * dk + j];
      P[(size_t)i * dk + j] = p;
    }
  }
}

/*
 * Generic recurrence: S_t = (D_t - A_t B_t^T) S_{t-1} + sum_r K_{t,r} V_{t,r}^T,
 * o_t = S_t^T q_t (state after token t's update).
 * out may be NULL (no readout); Sfin may be NULL; S0 NULL means zero state.
 */
int oracle_generic(int64_t BH, int64_t T, int dk, int dv, int r_ab, int r_kv, int scalar_decay,
                   const double* q, const double* K, const double* V, const double* ld,
                   const double* A, const double* B, const double* S0, double* out,
                   double* Sfin, int nthreads) {
  if (BH < 0 || T < 0 || dk <= 0 || dv <= 0 || r_ab < 0 || r_kv < 0) return ORACLE_EINVAL;
  set_threads(nthreads);
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* P = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    if (!P || !S || !tmp) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < BH; ++bh) {
        if (S0) memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        for (int64_t t = 0; t < T; ++t) {
          const size_t tok = (size_t)bh * T + t;
          const double* ldt = scalar_decay ? ld + tok : ld + tok * dk;
          const double* At = r_ab ? A + tok * r_ab * dk : NULL;
          const double* Bt = r_ab ? B + tok * r_ab * dk : NULL;
          form_generic_P(dk, r_ab, scalar_decay, ldt, At, Bt, P);
          apply_left(dk, dv, P, S, tmp);
          for (int r = 0; r < r_kv; ++r) {
            const double* kr = K + (tok * r_kv + r) * dk;
            const double* vr = V + (tok * r_kv + r) * dv;
            for (int i = 0; i < dk; ++i)
              for (int c = 0; c < dv; ++c) S[(size_t)i * dv + c] += kr[i] * vr[c];
          }
          if (out) readout(dk, dv, S, q + tok * dk, out + tok * dv);
        }
        if (Sfin) memcpy(Sfin + (size_t)bh * dk * dv, S, sizeof(double) * (size_t)dk * dv);
      }
    }
    free(P); free(S); free(tmp);
  }
  return err;
}

/*
 * HDLA in its own (Householder) form, never touching A, B:
 *   H_t = I - beta_t k_t k_t^T,  P_t = H_t Diag(lambda_t) H_t,  lambda_t = exp(log_lambda_t)
 *   S_t = P_t S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
 * (HDLA note, "Key design 2": the Householder congruence decay; the write
 * beta_t k_t v_t^T is the delta-rule step of its test-time-training reading.)
 * k, q [BH,T,dk]; v [BH,T,dv]; log_lambda [BH,T,dk]; beta [BH,T].
 */
int oracle_hdla(int64_t BH, int64_t T, int dk, int dv, const double* q, const double* k,
                const double* v, const double* log_lambda, const double* beta,
                const double* S0, double* out, double* Sfin, int nthreads) {
  if (BH < 0 || T < 0 || dk <= 0 || dv <= 0) return ORACLE_EINVAL;
  set_threads(nthreads);
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* H = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    double* HL = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    double* P = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    if (!H || !HL || !P || !S || !tmp) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < BH; ++bh) {
        if (S0) memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        for (int64_t t = 0; t < T; ++t) {
          const size_t tok = (size_t)bh * T + t;
          const double* kt = k + tok * dk;
          const double* lt = log_lambda + tok * dk;
          const double bt = beta[tok];
          for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dk; ++j)
              H[(size_t)i * dk + j] = (i == j ? 1.0 : 0.0) - bt * kt[i] * kt[j];
          /* HL = H Diag(lambda) */
          for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dk; ++j) HL[(size_t)i * dk + j] = H[(size_t)i * dk + j] * exp(lt[j]);
          /* P = HL H */
          for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dk; ++j) {
              double s = 0.0;
              for (int m = 0; m < dk; ++m) s += HL[(size_t)i * dk + m] * H[(size_t)m * dk + j];
              P[(size_t)i * dk + j] = s;
            }
          apply_left(dk, dv, P, S, tmp);
          const double* vt = v + tok * dv;
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) S[(size_t)i * dv + c] += bt * kt[i] * vt[c];
          if (out) readout(dk, dv, S, q + tok * dk, out + tok * dv);
        }
        if (Sfin) memcpy(Sfin + (size_t)bh * dk * dv, S, sizeof(double) * (size_t)dk * dv);
      }
    }
    free(H); free(HL); free(P); free(S); free(tmp);
  }
  return err;
}

/*
 * Gated DeltaNet in its own form (HLA note, "Prerequisites: Gated DeltaNet"):
 *   P_t = exp(g_t) (I - beta_t k_t k_t^T),   S_t = P_t S_{t-1} + beta_t k_t v_t^T.
 * The page writes keys as row vectors; with column vectors the same update is
 * the one above.  g, beta [BH,T]; k, q [BH,T,dk]; v [BH,T,dv].
 */
int oracle_gdn(int64_t BH, int64_t T, int dk, int dv, const double* q, const double* k,
               const double* v, const double* g, const double* beta, const double* S0,
               double* out, double* Sfin, int nthreads) {
  if (BH < 0 || T < 0 || dk <= 0 || dv <= 0) return ORACLE_EINVAL;
  set_threads(nthreads);
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* P = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    if (!P || !S || !tmp) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < BH; ++bh) {
        if (S0) memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        for (int64_t t = 0; t < T; ++t) {
          const size_t tok = (size_t)bh * T + t;
          const double* kt = k + tok * dk;
          const double eg = exp(g[tok]);
          const double bt = beta[tok];
          for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dk; ++j)
              P[(size_t)i * dk + j] = eg * ((i == j ? 1.0 : 0.0) - bt * kt[i] * kt[j]);
          apply_left(dk, dv, P, S, tmp);
          const double* vt = v + tok * dv;
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) S[(size_t)i * dv + c] += bt * kt[i] * vt[c];
          if (out) readout(dk, dv, S, q + tok * dk, out + tok * dv);
        }
        if (Sfin) memcpy(Sfin + (size_t)bh * dk * dv, S, sizeof(double) * (size_t)dk * dv);
      }
    }
    free(P); free(S); free(tmp);
  }
  return err;
}

/*
 * Exact affine summary of every chunk (HLA note, "Affine maps and closure
 * under composition", and its remark on computing the pair jointly): run the
 * generic recurrence over the chunk's tokens on the widened state
 * Sigma = [B_j | A_j] (dk x (dv+dk)), starting from [0 | I], with values
 * [V_t | 0].  Afterwards S_j = A_j S_{j-1} + B_j for any incoming S_{j-1}.
 * Chunks are consecutive runs of `chunk` tokens; the last may be shorter.
 *   sumA [BH, N, dk, dk]   sumB [BH, N, dk, dv]   with N = ceil(T / chunk).
 */
int oracle_chunk_summaries(int64_t BH, int64_t T, int dk, int dv, int r_ab, int r_kv,
                           int scalar_decay, int chunk, const double* K, const double* V,
                           const double* ld, const double* A, const double* B, double* sumA,
                           double* sumB, int nthreads) {
  if (BH < 0 || T < 0 || dk <= 0 || dv <= 0 || chunk <= 0 || r_ab < 0 || r_kv < 0)
    return ORACLE_EINVAL;
  set_threads(nthreads);
  const int64_t N = (T + chunk - 1) / chunk;
  const int w = dv + dk;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* P = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    double* Sg = (double*)malloc(sizeof(double) * (size_t)dk * w);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)dk * w);
    if (!P || !Sg || !tmp) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    } else {
#pragma omp for collapse(2) schedule(dynamic, 1)
      for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t j = 0; j < N; ++j) {
          memset(Sg, 0, sizeof(double) * (size_t)dk * w);
          for (int i = 0; i < dk; ++i) Sg[(size_t)i * w + dv + i] = 1.0;
          const int64_t t1 = (j + 1) * chunk < T ? (j + 1) * chunk : T;
          for (int64_t t = j * chunk; t < t1; ++t) {
            const size_t tok = (size_t)bh * T + t;
            const double* ldt = scalar_decay ? ld + tok : ld + tok * dk;
            const double* At = r_ab ? A + tok * r_ab * dk : NULL;
            const double* Bt = r_ab ? B + tok * r_ab * dk : NULL;
            form_generic_P(dk, r_ab, scalar_decay, ldt, At, Bt, P);
            apply_left(dk, w, P, Sg, tmp);
            for (int r = 0; r < r_kv; ++r) {
              const double* kr = K + (tok * r_kv + r) * dk;
              const double* vr = V + (tok * r_kv + r) * dv;
              for (int i = 0; i < dk; ++i)
                for (int c = 0; c < dv; ++c) Sg[(size_t)i * w + c] += kr[i] * vr[c];
            }
          }
          double* oa = sumA + ((size_t)bh * N + j) * dk * dk;
          double* ob = sumB + ((size_t)bh * N + j) * dk * dv;
          for (int i = 0; i < dk; ++i) {
            for (int c = 0; c < dv; ++c) ob[(size_t)i * dv + c] = Sg[(size_t)i * w + c];
            for (int c = 0; c < dk; ++c) oa[(size_t)i * dk + c] = Sg[(size_t)i * w + dv + c];
          }
        }
      }
    }
    free(P); free(Sg); free(tmp);
  }
  return err;
}
