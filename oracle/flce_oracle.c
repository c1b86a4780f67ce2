/*
 * Oracle for the linear cross-entropy forward and its backward.
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it to check the GPU library; the library never calls
 * it.
 *
 * It is the plain definition from "Een gefuseerde forward-kernel
 * voor lineaire cross-entropy op Apple-GPU's" (section 1, the definition of plain
 * cross-entropy): with H an (N, D) matrix of hidden states and W a (V, D)
 * output projection, the logits are Z = H W^T and, for the target y_i,
 *     loss_i = logsumexp(Z_i) - Z_{i, y_i}.
 * The same section states that only two per-row statistics are needed, the
 * log-sum-exp and the target logit; both are returned.
 *
 * Each selected row is computed independently, in float64, with nothing
 * streamed or tiled: the V logits of the row are materialised in a buffer,
 * then the maximum M, then S = sum_v exp(z_v - M) in vocabulary order, then
 * lse = M + ln S and loss = lse - z_y. (The shift by M is the textbook
 * two-pass form of logsumexp; it changes nothing in exact arithmetic.)
 *
 * Readings where the page is silent:
 *   - the logarithm is natural (the page writes exp and logsumexp);
 *   - a target outside [0, V) has no defined loss: loss = NaN, lse is still
 *     returned and z_target = NaN;
 *   - there is no bias, scale, softcap, smoothing or reduction over rows.
 *
 * Inputs are the exact bit patterns the GPU reads: bfloat16 (dtype 0) or
 * IEEE fp32 (dtype 1), row-major, D contiguous. Each element is widened
 * exactly to double; products of two such values are exact in double, so the
 * only rounding is the float64 summation.
 *
 * Rows run in parallel with OpenMP; every row is still the same sequential
 * computation whatever the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) {
    uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * The V logits of row i, Z_i = H_i W^T, into z[0..V), and logsumexp(Z_i)
 * in two passes: the maximum, then the shifted sum.
 */
static double row_logits_lse(const void* H, const void* W, int64_t D, int64_t V, int dtype,
                             int64_t i, double* z) {
  for (int64_t v = 0; v < V; ++v) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d)
      acc += widen(H, dtype, i * D + d) * widen(W, dtype, v * D + d);
    z[v] = acc;
  }
  double M = z[0];
  for (int64_t v = 1; v < V; ++v)
    if (z[v] > M || isnan(z[v])) M = z[v];
  double S = 0.0;
  for (int64_t v = 0; v < V; ++v) S += exp(z[v] - M);
  double l = M + log(S);
  return l;
}

/*
 * rows: R row indices into [0, N) (NULL means rows 0..N-1 with R = N).
 * Writes loss[r], lse[r], z_target[r] for r in [0, R).
 * Returns 0, or -1 on an invalid argument or a failed allocation.
 */
int oracle_lce_forward(const void* H, const void* W, const int32_t* y,
                       int64_t N, int64_t D, int64_t V, int dtype,
                       const int64_t* rows, int64_t R,
                       double* loss, double* lse, double* z_target) {
  if (N < 0 || D < 1 || V < 1 || R < 0 || (dtype != 0 && dtype != 1)) return -1;
  if (!rows) R = N;
  if (R > 0 && (!H || !W || !y || !loss || !lse || !z_target)) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc((size_t)V * sizeof(double));
    if (!z) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
      if (!z) continue;
      int64_t i = rows ? rows[r] : r;
      if (i < 0 || i >= N) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const double l = row_logits_lse(H, W, D, V, dtype, i, z);
      lse[r] = l;
      int64_t t = (int64_t)y[i];
      if (t >= 0 && t < V) {
        z_target[r] = z[t];
        loss[r] = l - z[t];
      } else {
        z_target[r] = NAN;
        loss[r] = NAN;
      }
    }
    free(z);
  }
  return failed ? -1 : 0;
}

/*
 * Backward of the same definition, for an upstream gradient g (one value per
 * token): the gradient of sum_i g_i loss_i. The page's training path keeps
 * the forward log-sum-exp and regenerates the logits for its backward
 * (section 1); the derivative itself is the chain rule applied to the
 * definition above:
 *     p_iv   = exp(z_iv - lse_i)                  (softmax of row i)
 *     dZ_iv  = g_i (p_iv - [v == y_i])
 *     dH_i   = sum_v dZ_iv W_v                    (N x D)
 *     dW_v   = sum_i dZ_iv H_i                    (V x D)
 * Reading where the page is silent: a target outside [0, V) matches no v, so
 * that row contributes g_i p_i (the gradient of its lse alone); a caller that
 * ignores such rows passes g_i = 0.
 *
 * Everything is float64, row by row, with the row's logits materialised; lse
 * is recomputed here (two passes, as in the forward) rather than taken from
 * anywhere else. Alongside each output the sum of the absolute values of its
 * terms is returned, with dZ written as the two terms g_i p_iv and
 * -g_i [v == y_i]: dH_abs_id = sum_v |g_i| (p_iv + [v == y_i]) |W_vd| and
 * dW_abs_vd = sum_i |g_i| (p_iv + [v == y_i]) |H_id|. An evaluation that
 * rounds dZ, or computes p with a small relative error, is off by at most
 * that relative error times these sums.
 *
 * rows: R row indices for dH (NULL: all N rows, R = N). dW (and dW_abs) need
 * every row and are computed only when dW is not NULL; that keeps the N x V
 * matrix dZ in memory, so it is for small shapes.
 */
/* dZ_i = g_i (softmax(Z_i) - onehot(y_i)) into dz[0..V), and the absolute
 * size of its two terms, |g_i| (p_iv + [v == y_i]), into dzabs[0..V). */
static void row_dz(const void* H, const void* W, const int32_t* y, const double* g,
                   int64_t D, int64_t V, int dtype, int64_t i, double* dz, double* dzabs) {
  const double l = row_logits_lse(H, W, D, V, dtype, i, dz);
  const int64_t t = (int64_t)y[i];
  for (int64_t v = 0; v < V; ++v) {
    const double p = exp(dz[v] - l);
    const double hit = v == t ? 1.0 : 0.0;
    dz[v] = g[i] * (p - hit);
    dzabs[v] = fabs(g[i]) * (p + hit);
  }
}

int oracle_lce_backward(const void* H, const void* W, const int32_t* y, const double* g,
                        int64_t N, int64_t D, int64_t V, int dtype,
                        const int64_t* rows, int64_t R,
                        double* dH, double* dH_abs, double* dW, double* dW_abs) {
  if (N < 0 || D < 1 || V < 1 || R < 0 || (dtype != 0 && dtype != 1)) return -1;
  if (!rows) R = N;
  if (N > 0 && (!H || !W || !y || !g)) return -1;
  if (R > 0 && !dH) return -1;
  /* dZ and its term sizes for every row, when dW is wanted */
  double* dz_all = NULL;
  double* dzabs_all = NULL;
  if (dW) {
    const size_t n = (size_t)(N > 0 ? N : 1) * (size_t)V;
    dz_all = (double*)malloc(n * sizeof(double));
    dzabs_all = (double*)malloc(n * sizeof(double));
    if (!dz_all || !dzabs_all) {
      free(dz_all);
      free(dzabs_all);
      return -1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < N; ++i) row_dz(H, W, y, g, D, V, dtype, i, dz_all + i * V, dzabs_all + i * V);
  }
  int failed = 0;
  /* dH for the selected rows */
#pragma omp parallel
  {
    double* z = dz_all ? NULL : (double*)malloc(2 * (size_t)V * sizeof(double));
    if (!dz_all && !z) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
      if (!dz_all && !z) continue;
      const int64_t i = rows ? rows[r] : r;
      if (i < 0 || i >= N) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const double* dz = dz_all ? dz_all + i * V : z;
      const double* dzabs = dz_all ? dzabs_all + i * V : z + V;
      if (!dz_all) row_dz(H, W, y, g, D, V, dtype, i, z, z + V);
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0, aabs = 0.0;
        for (int64_t v = 0; v < V; ++v) {
          const double w = widen(W, dtype, v * D + d);
          acc += dz[v] * w;  /* dZ_iv W_vd */
          aabs += dzabs[v] * fabs(w);
        }
        dH[r * D + d] = acc;
        if (dH_abs) dH_abs[r * D + d] = aabs;
      }
    }
    free(z);
  }
  /* dW, every vocabulary row, summing over tokens in order */
  if (dW && !failed) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t v = 0; v < V; ++v) {
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0, aabs = 0.0;
        for (int64_t i = 0; i < N; ++i) {
          const double h = widen(H, dtype, i * D + d);
          acc += dz_all[i * V + v] * h;  /* dZ_iv H_id */
          aabs += dzabs_all[i * V + v] * fabs(h);
        }
        dW[v * D + d] = acc;
        if (dW_abs) dW_abs[v * D + d] = aabs;
      }
    }
  }
  free(dz_all);
  free(dzabs_all);
  return failed ? -1 : 0;
}
