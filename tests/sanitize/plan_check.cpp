// CPU check of the host planners (linear_cross_entropy_amd/csrc/flce_plan.h),
// built with the address and undefined-behaviour sanitizers by
// tests/test_sanitizers.py. Every planner runs over the shapes the tests and
// workloads use, random shapes, and extreme or invalid sizes; for each plan
// it accepts, the invariants the kernels rely on are checked. Exit status 0
// when all hold; otherwise the first failure is printed.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "flce_plan.h"

using namespace flce_plan;

static int failures = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                       \
      fprintf(stderr, "\n");                              \
      ++failures;                                         \
      return;                                             \
    }                                                     \
  } while (0)

static bool aligned256(size_t x) { return x % 256 == 0; }

static void check_forward(int64_t N, int64_t D, int64_t V, int dtype) {
  Plan pl;
  const int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return;
  const int64_t es = dtype == FLCE_BF16 ? 2 : 4;
  CHECK(pl.row_bytes == D * es, "row bytes N=%lld D=%lld V=%lld", (long long)N, (long long)D, (long long)V);
  CHECK((int64_t)pl.row_blocks * pl.BT >= N && (pl.row_blocks - 1) * (int64_t)pl.BT < (N > 0 ? N : 1),
        "row blocks N=%lld", (long long)N);
  CHECK((int64_t)pl.vocab_tiles * pl.BV >= V && (int64_t)(pl.vocab_tiles - 1) * pl.BV < V, "vocab tiles V=%lld",
        (long long)V);
  CHECK(pl.chunks >= 1 && pl.chunks <= pl.vocab_tiles, "chunks %d of %d tiles", pl.chunks, pl.vocab_tiles);
  const int64_t per = (pl.vocab_tiles + pl.chunks - 1) / pl.chunks;
  CHECK(per * pl.BV * (int64_t)pl.row_bytes < (int64_t(1) << 31), "chunk resource N=%lld D=%lld V=%lld",
        (long long)N, (long long)D, (long long)V);
  CHECK(pl.grid == (pl.row_blocks > 0 ? pl.row_blocks : 1) * pl.chunks, "grid");
  CHECK(pl.lds_bytes <= 160 * 1024 && (pl.threads == 512), "tile resources");
  CHECK(aligned256(pl.off_s) && aligned256(pl.off_z) && aligned256(pl.ws_bytes), "workspace alignment");
  CHECK(pl.off_s >= (size_t)pl.chunks * N * 4 && pl.off_z >= pl.off_s + (size_t)pl.chunks * N * 4 &&
            pl.ws_bytes >= pl.off_z + (size_t)N * 4,
        "workspace layout");
  if (pl.xcd_rows > 0) {
    // the kernel's workgroup -> (row block, chunk) remap must be a bijection
    const int RB = pl.row_blocks, C = pl.chunks;
    CHECK(RB % pl.xcd_rows == 0 && C % pl.xcd_chunks == 0 && pl.grid % 8 == 0, "xcd groups");
    const int gc = C / pl.xcd_chunks;
    char* seen = (char*)calloc((size_t)pl.grid, 1);
    for (int b = 0; b < pl.grid; ++b) {
      const int x = b & 7, j = b >> 3;
      const int rb = (x / gc) * pl.xcd_rows + j / pl.xcd_chunks;
      const int ch = (x % gc) * pl.xcd_chunks + j % pl.xcd_chunks;
      if (rb < 0 || rb >= RB || ch < 0 || ch >= C || seen[rb * C + ch]) {
        free(seen);
        CHECK(false, "xcd remap not a bijection at %d", b);
      }
      seen[rb * C + ch] = 1;
    }
    free(seen);
  }
}

static void check_backward(int64_t N, int64_t D, int64_t V, int dtype) {
  BwdPlan bp;
  if (make_bwd_plan(N, D, V, dtype, &bp) != FLCE_OK) return;
  const int64_t es = dtype == FLCE_BF16 ? 2 : 4;
  CHECK(bp.Np % 64 == 0 && bp.Np >= N, "Np");
  if (N == 0) {
    CHECK(bp.slices == 0, "no slices without rows");
    return;
  }
  CHECK(bp.Vs >= 1 && (int64_t)bp.slices * bp.Vs >= V && (int64_t)(bp.slices - 1) * bp.Vs < V,
        "slices cover V=%lld", (long long)V);
  CHECK(bp.last.Vs == V - (int64_t)(bp.slices - 1) * bp.Vs && bp.last.Vs >= 1, "last slice");
  CHECK(bp.full.Vsp % 64 == 0 && bp.full.Vsp >= bp.full.Vs && bp.last.Vsp <= bp.full.Vsp, "slice padding");
  const double dz = (double)bp.full.Vsp * (double)bp.Np * (double)es * (dtype == FLCE_BF16 ? 1 : 2);
  if (bp.Vs > 64) CHECK(dz <= kDzBudget + 64.0 * bp.Np * es * 2, "dZ budget N=%lld V=%lld", (long long)N, (long long)V);
  CHECK(bp.full.ksplit >= 1 && bp.full.ksplit <= 16 && bp.last.ksplit >= 1 && bp.last.ksplit <= 16, "ksplit");
  CHECK(aligned256(bp.off_ht) && aligned256(bp.off_dzt) && aligned256(bp.off_dz) && aligned256(bp.off_part) &&
            aligned256(bp.ws_bytes),
        "workspace alignment");
  CHECK(bp.off_ht >= (size_t)(D * bp.full.Vsp * es) && bp.off_dzt >= bp.off_ht + (size_t)(D * bp.Np * es) &&
            bp.off_dz >= bp.off_dzt + (size_t)(bp.full.Vsp * bp.Np * es) && bp.ws_bytes >= bp.off_part,
        "workspace layout");
}

static void check_quant(int64_t N, int64_t D, int64_t V, int bits, int group) {
  QuantPlan qp;
  if (make_quant_plan(N, D, V, bits, group, &qp) == FLCE_OK) {
    CHECK(qp.slices >= 1 && (int64_t)qp.slices * qp.Vs >= V && (int64_t)(qp.slices - 1) * qp.Vs < V, "quant slices");
    CHECK(qp.chunks_total == (qp.slices - 1) * qp.full.chunks + qp.last.chunks, "quant chunks");
    CHECK(aligned256(qp.off_m) && aligned256(qp.off_s) && aligned256(qp.off_z) && aligned256(qp.ws_bytes),
          "quant alignment");
  }
  QuantBwdPlan qb;
  if (N > 0 && make_quant_bwd_plan(N, D, V, bits, group, &qb) == FLCE_OK) {
    CHECK(qb.slices >= 1 && (int64_t)qb.slices * qb.Vs >= V && (int64_t)(qb.slices - 1) * qb.Vs < V,
          "quant bwd slices");
    CHECK(qb.Vs <= qp.Vs, "quant bwd slice within the forward's");
    CHECK(aligned256(qb.off_wt) && aligned256(qb.off_dzt) && aligned256(qb.off_part) && aligned256(qb.ws_bytes),
          "quant bwd alignment");
  }
}

static void check_all(int64_t N, int64_t D, int64_t V) {
  for (int dt = -1; dt <= 2; ++dt) {
    check_forward(N, D, V, dt);
    check_backward(N, D, V, dt);
  }
  for (int bits : {4, 8, 5})
    for (int group : {8, 32, 64, 20, 0, -8}) check_quant(N, D, V, bits, group);
}

int main() {
  const int64_t big = int64_t(1) << 40;
  const int64_t shapes[][3] = {
      {128, 64, 1024},     {2048, 1024, 32000},   {4096, 2048, 50257},  {8192, 4096, 151936},
      {8192, 8192, 262144}, {1, 8, 1},            {3, 8, 2},            {3, 72, 31},
      {257, 72, 255},      {300, 4104, 513},      {1000, 136, 100003},  {4096, 64, 65536},
      {3000, 64, 120000},  {5000, 64, 262144},    {1, 2097152, 257},    {1, 1048576, 257},
      {0, 8, 10},          {4, 12, 10},           {-1, 8, 10},          {4, 0, 10},
      {4, 8, 0},           {INT32_MAX, 8, 10},    {INT32_MAX / 2, 8, 10}, {8, 8, INT32_MAX},
      {8, INT32_MAX, 8},   {big, 4096, 151936},   {8192, big, 151936},  {8192, 4096, big},
      {65536, 4096, 151936}, {262144, 4096, 151936}, {1 << 22, 4096, 151936}, {32, 1 << 24, 64},
  };
  for (const auto& s : shapes) check_all(s[0], s[1], s[2]);
  // seeded random shapes, log-uniform over the ranges the library serves
  uint64_t x = 0x9E3779B97F4A7C15ull;
  auto next = [&]() {
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return x;
  };
  for (int i = 0; i < 1000; ++i) {
    const int64_t N = (int64_t)(next() % 20000);
    const int64_t D = 8 * (1 + (int64_t)(next() % 2048));
    const int64_t V = 1 + (int64_t)(next() % 300000);
    check_all(N, D, V);
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("plan_check ok\n");
  return 0;
}
