/*
 * CPU check of the float64 oracle (oracle/flce_oracle.c) under the address
 * and undefined-behaviour sanitizers, built by tests/test_sanitizers.py. It
 * runs the oracle's forward and backward on small seeded inputs in both
 * element types, with row subsets, a batch of zero rows, a vocabulary of one,
 * targets outside [0, V), a NaN input and rejected arguments, and checks the
 * results for what holds whatever the inputs (finite where they must be,
 * loss >= 0 for valid targets, NaN where the definition has no value, dH of a
 * row subset equal to those rows of the full run). Exit status 0 when all
 * hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_lce_forward(const void* H, const void* W, const int32_t* y, int64_t N, int64_t D, int64_t V, int dtype,
                       const int64_t* rows, int64_t R, double* loss, double* lse, double* z_target);
int oracle_lce_backward(const void* H, const void* W, const int32_t* y, const double* g, int64_t N, int64_t D,
                        int64_t V, int dtype, const int64_t* rows, int64_t R, double* dH, double* dH_abs,
                        double* dW, double* dW_abs);

static int failures = 0;
#define CHECK(c, msg)                                          \
  do {                                                         \
    if (!(c)) {                                                \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, msg); \
      ++failures;                                              \
    }                                                          \
  } while (0)

static uint64_t state = 0x243F6A8885A308D3ull;
static double uniform(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / 9007199254740992.0;
}
static double normal(void) {
  const double u = uniform() + 1e-12, v = uniform();
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* Inputs of one case, in the element type (0: bf16 bits, 1: float). */
static void* make(int64_t n, int dtype, double scale) {
  void* p = malloc((size_t)(n > 0 ? n : 1) * (dtype == 0 ? 2 : 4));
  for (int64_t i = 0; i < n; ++i) {
    const float f = (float)(normal() * scale);
    if (dtype == 0) ((uint16_t*)p)[i] = to_bf16(f);
    else ((float*)p)[i] = f;
  }
  return p;
}

static void run_case(int64_t N, int64_t D, int64_t V, int dtype) {
  void* H = make(N * D, dtype, 1.0);
  void* W = make(V * D, dtype, 0.5);
  int32_t* y = (int32_t*)malloc((size_t)(N > 0 ? N : 1) * 4);
  double* g = (double*)malloc((size_t)(N > 0 ? N : 1) * 8);
  for (int64_t i = 0; i < N; ++i) {
    y[i] = (int32_t)(uniform() * (double)V);
    g[i] = uniform() * 2.0 - 0.5;
  }
  if (N > 2) {
    y[1] = -1;          /* outside [0, V): NaN loss, valid lse */
    y[2] = (int32_t)V;
  }
  const size_t n1 = (size_t)(N > 0 ? N : 1);
  double* loss = (double*)malloc(n1 * 8);
  double* lse = (double*)malloc(n1 * 8);
  double* zt = (double*)malloc(n1 * 8);
  CHECK(oracle_lce_forward(H, W, y, N, D, V, dtype, NULL, N, loss, lse, zt) == 0, "forward rejected");
  for (int64_t i = 0; i < N; ++i) {
    const int valid = y[i] >= 0 && y[i] < V;
    CHECK(isfinite(lse[i]), "lse not finite");
    CHECK(valid ? (loss[i] >= -1e-12 && isfinite(loss[i])) : isnan(loss[i]), "loss");
  }
  /* a row subset in another order */
  if (N > 3) {
    int64_t rows[3] = {N - 1, 0, N / 2};
    double l2[3], s2[3], z2[3];
    CHECK(oracle_lce_forward(H, W, y, N, D, V, dtype, rows, 3, l2, s2, z2) == 0, "subset rejected");
    for (int k = 0; k < 3; ++k) CHECK(s2[k] == lse[rows[k]], "subset lse differs");
  }
  /* backward: all rows with dW, then a subset without */
  const size_t nd = (size_t)(N > 0 ? N : 1) * (size_t)D, vd = (size_t)V * (size_t)D;
  double* dH = (double*)malloc(nd * 8);
  double* dHa = (double*)malloc(nd * 8);
  double* dW = (double*)malloc(vd * 8);
  double* dWa = (double*)malloc(vd * 8);
  CHECK(oracle_lce_backward(H, W, y, g, N, D, V, dtype, NULL, N, dH, dHa, dW, dWa) == 0, "backward rejected");
  for (size_t k = 0; k < (size_t)N * (size_t)D; ++k) CHECK(isfinite(dH[k]) && dHa[k] >= fabs(dH[k]), "dH");
  for (size_t k = 0; k < vd; ++k) CHECK(isfinite(dW[k]) && dWa[k] >= fabs(dW[k]), "dW");
  if (N > 3) {
    int64_t rows[2] = {N - 1, 1};
    double* sub = (double*)malloc(2 * (size_t)D * 8);
    double* suba = (double*)malloc(2 * (size_t)D * 8);
    CHECK(oracle_lce_backward(H, W, y, g, N, D, V, dtype, rows, 2, sub, suba, NULL, NULL) == 0, "bwd subset");
    for (int64_t d = 0; d < D; ++d) {
      CHECK(sub[d] == dH[(N - 1) * D + d] && sub[D + d] == dH[D + d], "bwd subset differs");
    }
    free(sub);
    free(suba);
  }
  free(H); free(W); free(y); free(g); free(loss); free(lse); free(zt);
  free(dH); free(dHa); free(dW); free(dWa);
}

int main(void) {
  const int64_t shapes[][3] = {{1, 1, 1}, {3, 8, 2}, {5, 16, 1}, {7, 9, 33}, {16, 24, 100}, {0, 8, 10}, {33, 5, 257}};
  for (int dt = 0; dt < 2; ++dt)
    for (size_t k = 0; k < sizeof shapes / sizeof shapes[0]; ++k) run_case(shapes[k][0], shapes[k][1], shapes[k][2], dt);
  /* a NaN input reaches only its own row */
  {
    float H[2 * 4] = {1, 2, 3, 4, 1, 1, 1, 1}, W[3 * 4] = {0};
    int32_t y[2] = {0, 1};
    double loss[2], lse[2], zt[2];
    H[1] = NAN;
    CHECK(oracle_lce_forward(H, W, y, 2, 4, 3, 1, NULL, 2, loss, lse, zt) == 0, "nan case rejected");
    CHECK(isnan(lse[0]) && isnan(loss[0]) && fabs(lse[1] - log(3.0)) < 1e-15, "nan row");
  }
  /* rejected arguments */
  {
    double out[4];
    float h[4] = {0};
    int32_t y[1] = {0};
    int64_t bad_row[1] = {5};
    CHECK(oracle_lce_forward(NULL, NULL, NULL, 1, 0, 1, 0, NULL, 0, out, out, out) == -1, "D = 0");
    CHECK(oracle_lce_forward(NULL, NULL, NULL, 1, 1, 0, 0, NULL, 0, out, out, out) == -1, "V = 0");
    CHECK(oracle_lce_forward(NULL, NULL, NULL, 1, 1, 1, 7, NULL, 0, out, out, out) == -1, "dtype");
    CHECK(oracle_lce_forward(h, h, y, 1, 1, 1, 1, bad_row, 1, out, out, out) == -1, "row out of range");
    double g[1] = {1};
    CHECK(oracle_lce_backward(h, h, y, g, 1, 1, 1, 1, bad_row, 1, out, out, NULL, NULL) == -1, "bwd row");
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle_check ok\n");
  return 0;
}
