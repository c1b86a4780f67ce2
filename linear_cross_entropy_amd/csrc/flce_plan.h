// Host-side planning of the fused linear cross-entropy launches: tile
// configurations, the split of the (row block, vocabulary chunk) grid, the
// workspace layouts of the forward, the backward's vocabulary slices and the
// quantised head's slices. Plain C++ (no HIP): the GPU library includes it,
// and so does a CPU-only check built with the address and undefined-behaviour
// sanitizers, which exercises these planners over many shapes.
#ifndef FLCE_PLAN_H
#define FLCE_PLAN_H

#include <algorithm>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include "flce.h"

namespace flce_plan {

// ------------------------------------------------------------------ tiles
// A tile configuration: BV vocabulary rows x BT tokens per workgroup, split
// over WAVES_V x WAVES_T waves; each wave owns a (BV/WAVES_V) x (BT/WAVES_T)
// block of M x M MFMA tiles (M = 32: v_mfma_f32_32x32x16_bf16, K = 16 per
// instruction; M = 16: v_mfma_f32_16x16x32_bf16, K = 32). K is staged 128
// bytes (64 bf16 / 32 fp32) at a time, double-buffered in LDS; every wave
// fills BV/NW W rows and BT/NW H rows of each stage.
constexpr int kStageRowBytes = 128;

template <int BV_, int BT_, int WAVES_V_, int WAVES_T_, int M_ = 32>
struct TileCfg {
  static constexpr int BV = BV_, BT = BT_, WAVES_V = WAVES_V_, WAVES_T = WAVES_T_, M = M_;
  static constexpr int NW = WAVES_V * WAVES_T;
  static constexpr int THREADS = 64 * NW;
  static constexpr int WV = BV / WAVES_V;          // vocabulary rows per wave
  static constexpr int WT = BT / WAVES_T;          // tokens per wave
  static constexpr int MB = WV / M;                // M x M MFMA tiles along vocabulary
  static constexpr int NB = WT / M;                // ... and along tokens
  static constexpr int KSTEPS = M / 8;             // MFMA K steps per 128-byte stage (bf16): 4 or 2
  static constexpr int ACC = M * M / 64;           // accumulator registers per lane and MFMA tile
  static constexpr int WROWS = BV / NW;            // W rows each wave fills per stage
  static constexpr int HROWS = BT / NW;            // H rows each wave fills per stage
  static constexpr int WLOADS = WROWS / 8;         // 16-byte loads per lane (8 rows each)
  static constexpr int HLOADS = HROWS / 8;
  static constexpr int STAGE_BYTES = (BV + BT) * kStageRowBytes;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  // Whether the younger wave of each SIMD takes issue priority around the
  // stage barrier (see the main loop). Measured on the production shape: the
  // 256-row 32x32 tile is 3% faster with it, the 320- and 384-row 32x32 tiles
  // up to 1% faster without it, and the 320-row 16x16 tile 1.3% faster
  // without it.
  static constexpr bool YOUNG_PRIO = BV == 256;
  static_assert(M == 32 || M == 16, "MFMA shape");
  static_assert(WV % M == 0 && WT % M == 0, "waves own whole MFMA tiles");
  static_assert(WROWS % 8 == 0 && HROWS % 8 == 0 && BV % 16 == 0, "whole 8-row loads");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS");
};
// All run 8 waves (two per SIMD). Staged bytes per FLOP fall with the tile,
// (BV + BT) / (BV * BT): 256x256 stages 512 rows per 65536 logits, 320x256
// 576 per 81920 (-10%), 384x256 640 per 98304 (-17%); 384x256 takes the whole
// 160 KB of LDS and 192 accumulator registers per lane.
//
// The MFMA shape matters as much. The part holds its power limit by lowering
// the clock, and with random operands the 16x16x32 bf16 instruction runs at a
// ~15% higher clock than the 32x32x16 one for the same FLOP (less register
// traffic per FLOP: a quarter of the accumulator bytes per instruction for
// half the FLOP). Measured on the production shape, one box, alternating
// launches: 384x256 with 32x32 tiles 6.93 ms; 320x256 with 16x16 tiles 6.70
// ms; 256x256 with 16x16 7.02 ms, with 32x32 7.29 ms. The 16x16 shape holds
// four token columns per lane instead of two (more B fragments and more
// per-token state), so at 384x256 it no longer fits the register file
// without spilling in the stage loop: the bf16 tiles are 256x256 and
// 320x256 with 16x16 MFMAs and 384x256 with 32x32 ones. fp32 and the
// transposed-B product run 32x32 tiles.
typedef TileCfg<256, 256, 2, 4> Tile256;        // 32x32: fp32, and the transposed-B dH product
typedef TileCfg<320, 256, 2, 4> Tile320;        // 32x32: the transposed-B dH product
typedef TileCfg<384, 256, 2, 4> Tile384;        // 32x32
typedef TileCfg<256, 256, 2, 4, 16> Tile256h;   // 16x16
typedef TileCfg<320, 256, 2, 4, 16> Tile320h;   // 16x16


// ------------------------------------------------------------------ forward plan
constexpr int kSlots = 256;       // workgroups resident at once: one per CU
constexpr size_t kAlign = 256;

enum TileId { kTile256 = 0, kTile320 = 1, kTile384 = 2 };

struct Plan {
  int N, V, row_bytes, dtype, tile;
  int BV, BT, threads, lds_bytes;
  int row_blocks, vocab_tiles, chunks, grid, xcd_rows, xcd_chunks;
  size_t off_m, off_s, off_z, ws_bytes;
};

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct TileInfo {
  int BV, BT, threads, lds_bytes;
  int cost_per_logit;  // relative time per logit at large shapes (x1000), measured on MI355X
};
template <typename C>
constexpr TileInfo tile_info(int cost) {
  return TileInfo{C::BV, C::BT, C::THREADS, C::LDS_BYTES, cost};
}
// Per-logit costs of the bf16 tiles from the production shape (N=8192,
// D=4096, V=151936), one box, alternating launches: 7.02 ms (256x256, 16x16
// MFMAs), 6.70 ms (320x256, 16x16) and 6.93 ms (384x256, 32x32) for the same
// work. The geometry (BV, BT, threads, LDS) of a tile id is the same for
// fp32, which runs 32x32 MFMAs on the 256x256 tile.
constexpr TileInfo kTiles[3] = {tile_info<Tile256h>(1048), tile_info<Tile320h>(1000), tile_info<Tile384>(1035)};
// The backward's launches (the dZ pass and the products) run 32x32 tiles at
// every size: its time goes to storing dZ and to the dH product rather than
// to the matrix cores' clock, and with 16x16 tiles it was no faster (25.95
// and 26.00 ms against 25.72 ms at the production shape). Their per-logit
// costs: 7.29, 7.13 and 7.05 ms for the same work with 256-, 320- and
// 384-row 32x32 tiles.
constexpr TileInfo kTilesM32[3] = {tile_info<Tile256>(1034), tile_info<Tile320>(1011), tile_info<Tile384>(1000)};

// Chunks per row block for a tile: minimise the makespan in tile-times,
// ceil(row_blocks*c / slots) * ceil(vocab_tiles / c); ties go to fewer chunks.
// Returns 0 when no chunk count keeps a chunk's W rows under 2^31 bytes.
inline int best_chunks(int64_t row_blocks, int64_t vocab_tiles, int64_t BV, int64_t row_bytes, int64_t* makespan) {
  int best_c = 0;
  int64_t best_cost = INT64_MAX;
  const int64_t RB = row_blocks > 0 ? row_blocks : 1;
  for (int64_t c = 1; c <= vocab_tiles; ++c) {
    const int64_t rounds = (RB * c + kSlots - 1) / kSlots;
    const int64_t per = (vocab_tiles + c - 1) / c;
    if (per * BV * row_bytes >= (int64_t(1) << 31)) continue;  // one buffer resource per chunk
    const int64_t cost = rounds * per;
    if (cost < best_cost) {
      best_cost = cost;
      best_c = (int)c;
    }
  }
  *makespan = best_cost;
  return best_c;
}

// Tile configuration for a shape: fp32 always uses 256x256; for bf16 the
// tile whose makespan (tile-times x logits per tile x cost per logit) is
// smallest. FLCE_TILE=256, 320 or 384 in the environment forces a bf16
// configuration (for tests and tuning; every configuration computes the same
// result). No tile above max_tile is chosen (forced ones included).
inline int choose_tile(int64_t N, int64_t V, int64_t row_bytes, int dtype, int max_tile, const TileInfo* tiles) {
  if (dtype != FLCE_BF16) return kTile256;
  static const int forced = [] {
    const char* e = getenv("FLCE_TILE");
    const int v = e ? atoi(e) : 0;
    return v == 256 ? kTile256 : v == 320 ? kTile320 : v == 384 ? kTile384 : -1;
  }();
  if (forced >= 0) return std::min(forced, max_tile);
  int best = kTile256;
  double best_t = 0;
  for (int t = kTile256; t <= max_tile; ++t) {
    const TileInfo& ti = tiles[t];
    int64_t makespan = 0;
    if (best_chunks((N + ti.BT - 1) / ti.BT, (V + ti.BV - 1) / ti.BV, ti.BV, row_bytes, &makespan) == 0) continue;
    const double est = (double)makespan * ti.BV * ti.BT * ti.cost_per_logit;
    if (t == kTile256 || est < best_t) {
      best = t;
      best_t = est;
    }
  }
  return best;
}

// m32: plan for 32x32-MFMA tiles (the backward's launches); otherwise for the
// forward's tiles (16x16 MFMAs at 256 and 320 rows).
inline int make_plan(int64_t N, int64_t D, int64_t V, int dtype, Plan* pl, int max_tile = kTile384,
                     bool m32 = false) {
  if (dtype != FLCE_BF16 && dtype != FLCE_FP32) return FLCE_ERR_UNSUPPORTED;
  if (N < 0 || D < 1 || V < 1) return FLCE_ERR_INVALID_ARG;
  // int32 indices and 32-bit buffer offsets: larger sizes are refused before
  // any planning (the chunk search below is linear in the vocabulary tiles)
  if (N > INT32_MAX / 2 || V > INT32_MAX - 384 || D > INT32_MAX / 4) return FLCE_ERR_UNSUPPORTED;
  const int64_t es = dtype == FLCE_BF16 ? 2 : 4;
  const int64_t rb = D * es;
  if (rb % 16 != 0) return FLCE_ERR_UNSUPPORTED;
  const TileInfo* tiles = m32 ? kTilesM32 : kTiles;
  pl->tile = choose_tile(N, V, rb, dtype, max_tile, tiles);
  const TileInfo& ti = tiles[pl->tile];
  const int kBV = ti.BV, kBT = ti.BT;
  pl->BV = kBV;
  pl->BT = kBT;
  pl->threads = ti.threads;
  pl->lds_bytes = ti.lds_bytes;
  // 32-bit offsets inside one tile's buffer resource, int32 indices elsewhere
  if ((int64_t)kBV * rb >= (int64_t(1) << 31) || N > INT32_MAX / 2 || V > INT32_MAX - kBV)
    return FLCE_ERR_UNSUPPORTED;
  pl->N = (int)N;
  pl->V = (int)V;
  pl->row_bytes = (int)rb;
  pl->dtype = dtype;
  pl->row_blocks = (int)((N + kBT - 1) / kBT);
  pl->vocab_tiles = (int)((V + kBV - 1) / kBV);
  int64_t makespan = 0;
  const int best_c = best_chunks(pl->row_blocks, pl->vocab_tiles, kBV, rb, &makespan);
  if (best_c == 0) return FLCE_ERR_UNSUPPORTED;
  const int RB = pl->row_blocks > 0 ? pl->row_blocks : 1;
  pl->chunks = best_c;
  pl->grid = RB * best_c;
  // XCD groups: 8 equal blocks of the (row block, chunk) grid, each
  // xcd_rows x xcd_chunks, chosen to minimise the distinct bytes of H and W
  // one XCD touches per tile-time (proportional to xcd_rows*BT + xcd_chunks*BV).
  pl->xcd_rows = 0;
  pl->xcd_chunks = 0;
  if (pl->grid % 8 == 0) {
    int64_t best = INT64_MAX;
    for (int gr = 1; gr <= RB; ++gr) {
      if (RB % gr) continue;
      const int per = pl->grid / 8;
      if (per % gr) continue;
      const int gc = per / gr;
      if (best_c % gc) continue;
      if ((RB / gr) * (best_c / gc) != 8) continue;
      const int64_t cost = (int64_t)gr * kBT + (int64_t)gc * kBV;
      if (cost < best) {
        best = cost;
        pl->xcd_rows = gr;
        pl->xcd_chunks = gc;
      }
    }
  }
  pl->off_m = 0;
  pl->off_s = align_up((size_t)best_c * N * sizeof(float));
  pl->off_z = pl->off_s + align_up((size_t)best_c * N * sizeof(float));
  pl->ws_bytes = pl->off_z + align_up((size_t)N * sizeof(float));
  return FLCE_OK;
}


// ------------------------------------------------------------------ backward plan
// (what the slices are: see the backward section of flce.hip)
constexpr double kDzBudget = 1024.0 * 1024 * 1024;

// The launches of one vocabulary slice of Vs rows.
struct SlicePlans {
  int64_t Vs, Vsp;
  Plan dz, dh, dw;     // dZ pass; dH product; dW product (dw unused when dW is not wanted)
  int ksplit, ks_per;  // bf16 dH: K slices and k-stages per slice
};

struct BwdPlan {
  int64_t N, D, V, Np, Vs;  // Vs: rows of every slice but the last
  int dtype, slices;
  size_t es;
  SlicePlans full, last;
  size_t off_wt, off_ht, off_dzt, off_dz, off_part, ws_bytes;
};

// K slices for the transposed-B dH product: when its tiles leave CUs idle,
// split the contraction over V so that up to kSlots workgroups run, keeping
// at least 16 k-stages (1024 of K) per slice and at most 16 slices.
inline void gemmt_split(const Plan& ph, int* ksplit, int* ks_per) {
  const int64_t grid = (int64_t)ph.row_blocks * ph.chunks;
  const int ks_all = (ph.row_bytes + kStageRowBytes - 1) / kStageRowBytes;
  int S = 1;
  while (S < 16 && grid * (S + 1) <= kSlots && ks_all / (S + 1) >= 16) ++S;
  const int per = (ks_all + S - 1) / S;
  *ks_per = per;
  *ksplit = (ks_all + per - 1) / per;
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Plans of one slice's launches (N > 0). with_dw: plan the dW product too.
inline int make_slice_plans(int64_t N, int64_t D, int64_t Vs, int64_t Np, int dtype, bool with_dw, SlicePlans* sp) {
  sp->Vs = Vs;
  sp->Vsp = round_up(Vs, 64);
  sp->ksplit = 1;
  sp->ks_per = 0;
  int rc;
  if ((rc = make_plan(N, D, Vs, dtype, &sp->dz, kTile384, true)) != FLCE_OK) return rc;                 // dZ
  if (dtype == FLCE_BF16) {
    if ((rc = make_plan(N, sp->Vsp, D, dtype, &sp->dh, kTile320, true)) != FLCE_OK) return rc;          // dH (transposed B)
    gemmt_split(sp->dh, &sp->ksplit, &sp->ks_per);
  } else {
    if ((rc = make_plan(D, sp->Vsp, N, dtype, &sp->dh, kTile384, true)) != FLCE_OK) return rc;          // dH
  }
  if (with_dw && (rc = make_plan(D, Np, Vs, dtype, &sp->dw, kTile384, true)) != FLCE_OK) return rc;    // dW
  return FLCE_OK;
}

// Vocabulary rows per slice: every slice's dZ (dz_copies copies of Vsp x Np
// elements) fits kDzBudget bytes, the slices are balanced, and a slice is a
// multiple of 6144 rows when that leaves at least one such block, else of 64:
// 6144 rows are 16 tiles of 384 (24 of 256), so the dZ pass and the dW
// product split a slice's tiles evenly over their 8 or 16 chunks (measured at
// the production shape: 23.95 ms a backward against 24.26 ms with 3840-row
// multiples; 23.72 ms without slices, i.e. with dZ for all rows).
inline int64_t slice_rows(int64_t V, int64_t Np, int64_t es, int dz_copies) {
  const int64_t cap = (int64_t)(kDzBudget / ((double)Np * (double)es * dz_copies));
  const int64_t gran = cap >= 6144 ? 6144 : 64;
  const int64_t maxv = std::max<int64_t>(cap / gran * gran, 64);
  if (V <= maxv) return V;
  const int64_t n = (V + maxv - 1) / maxv;
  return std::min(maxv, round_up((V + n - 1) / n, gran));
}

inline int make_bwd_plan(int64_t N, int64_t D, int64_t V, int dtype, BwdPlan* bp) {
  if (dtype != FLCE_BF16 && dtype != FLCE_FP32) return FLCE_ERR_UNSUPPORTED;
  if (N < 0 || D < 1 || V < 1) return FLCE_ERR_INVALID_ARG;
  const int64_t es = dtype == FLCE_BF16 ? 2 : 4;
  if ((D * es) % 16 != 0) return FLCE_ERR_UNSUPPORTED;
  if (N > INT32_MAX / 2 || V > INT32_MAX / 2 || D > INT32_MAX / 2) return FLCE_ERR_UNSUPPORTED;
  bp->N = N;
  bp->D = D;
  bp->V = V;
  bp->dtype = dtype;
  bp->es = (size_t)es;
  bp->Np = round_up(N, 64);
  // a stage of the transposed B (64 k-rows of dzt) stays under 2^31 bytes
  if (bp->Np * es * 64 >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;
  bp->Vs = slice_rows(V, bp->Np, es, dtype == FLCE_BF16 ? 1 : 2);
  bp->slices = N > 0 ? (int)((V + bp->Vs - 1) / bp->Vs) : 0;
  int rc;
  if (N > 0) {
    if ((rc = make_slice_plans(N, D, bp->Vs, bp->Np, dtype, true, &bp->full)) != FLCE_OK) return rc;
    if ((rc = make_slice_plans(N, D, V - (int64_t)(bp->slices - 1) * bp->Vs, bp->Np, dtype, true, &bp->last)) !=
        FLCE_OK)
      return rc;
  } else {
    bp->full.Vsp = bp->last.Vsp = 0;
    bp->full.ksplit = bp->last.ksplit = 1;
  }
  const int64_t vsp = bp->full.Vsp;
  if (vsp * es >= (int64_t(1) << 31) || bp->Np * es >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;
  const int parts = std::max(bp->full.ksplit, bp->last.ksplit);
  bp->off_wt = 0;
  bp->off_ht = align_up((size_t)(D * vsp * es));
  bp->off_dzt = bp->off_ht + align_up((size_t)(D * bp->Np * es));
  bp->off_dz = bp->off_dzt + align_up((size_t)(vsp * bp->Np * es));
  bp->off_part = bp->off_dz + (dtype == FLCE_BF16 ? 0 : align_up((size_t)(bp->Np * vsp * es)));
  bp->ws_bytes = bp->off_part + (parts > 1 ? align_up((size_t)parts * (size_t)(N * D) * 4) : 0);
  return FLCE_OK;
}


// ------------------------------------------------------------------ quantised head plans
constexpr double kQuantSliceBytes = 256.0 * 1024 * 1024;

struct QuantPlan {
  int64_t N, D, V, Vs;
  int bits, group, slices, chunks_total;
  Plan full, last;  // plans of a full slice and of the last one
  size_t off_buf, off_m, off_s, off_z, ws_bytes;
};

inline int make_quant_plan(int64_t N, int64_t D, int64_t V, int bits, int group, QuantPlan* qp) {
  if (N < 0 || D < 1 || V < 1) return FLCE_ERR_INVALID_ARG;
  if ((bits != 4 && bits != 8) || group < 8 || group % 8 != 0 || D % group != 0) return FLCE_ERR_UNSUPPORTED;
  qp->N = N;
  qp->D = D;
  qp->V = V;
  qp->bits = bits;
  qp->group = group;
  int64_t vs = (int64_t)(kQuantSliceBytes / (double)(D * 2)) / 3072 * 3072;
  if (vs < 3072) vs = 3072;
  qp->Vs = std::min(vs, V);
  qp->slices = (int)((V + qp->Vs - 1) / qp->Vs);
  int rc;
  if ((rc = make_plan(N, D, qp->Vs, FLCE_BF16, &qp->full)) != FLCE_OK) return rc;
  const int64_t v_last = V - (int64_t)(qp->slices - 1) * qp->Vs;
  if ((rc = make_plan(N, D, v_last, FLCE_BF16, &qp->last)) != FLCE_OK) return rc;
  if (V > INT32_MAX / 2) return FLCE_ERR_UNSUPPORTED;
  const int64_t C = (int64_t)(qp->slices - 1) * qp->full.chunks + qp->last.chunks;
  if (C > INT32_MAX) return FLCE_ERR_UNSUPPORTED;
  qp->chunks_total = (int)C;
  qp->off_buf = 0;
  qp->off_m = align_up((size_t)(qp->Vs * D * 2));
  qp->off_s = qp->off_m + align_up((size_t)C * N * sizeof(float));
  qp->off_z = qp->off_s + align_up((size_t)C * N * sizeof(float));
  qp->ws_bytes = qp->off_z + align_up((size_t)N * sizeof(float));
  return FLCE_OK;
}


struct QuantBwdPlan {
  int64_t N, D, V, Np, Vs;
  int bits, group, slices;
  SlicePlans full, last;
  size_t off_w, off_wt, off_dzt, off_part, ws_bytes;
};

inline int make_quant_bwd_plan(int64_t N, int64_t D, int64_t V, int bits, int group, QuantBwdPlan* qb) {
  int rc;
  QuantPlan q;
  if ((rc = make_quant_plan(N, D, V, bits, group, &q)) != FLCE_OK) return rc;
  qb->N = N;
  qb->D = D;
  qb->V = V;
  qb->bits = bits;
  qb->group = group;
  qb->Np = round_up(N, 64);
  if (qb->Np * 2 * 64 >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;
  qb->Vs = std::min(q.Vs, slice_rows(V, qb->Np, 2, 1));
  qb->slices = (int)((V + qb->Vs - 1) / qb->Vs);
  if ((rc = make_slice_plans(N, D, qb->Vs, qb->Np, FLCE_BF16, false, &qb->full)) != FLCE_OK) return rc;
  if ((rc = make_slice_plans(N, D, V - (int64_t)(qb->slices - 1) * qb->Vs, qb->Np, FLCE_BF16, false, &qb->last)) !=
      FLCE_OK)
    return rc;
  const int64_t vsp = qb->full.Vsp;
  const int parts = std::max(qb->full.ksplit, qb->last.ksplit);
  qb->off_w = 0;
  qb->off_wt = align_up((size_t)(qb->Vs * D * 2));
  qb->off_dzt = qb->off_wt + align_up((size_t)(D * vsp * 2));
  qb->off_part = qb->off_dzt + align_up((size_t)(vsp * qb->Np * 2));
  qb->ws_bytes = qb->off_part + (parts > 1 ? align_up((size_t)parts * (size_t)(N * D) * 4) : 0);
  return FLCE_OK;
}


}  // namespace flce_plan

#endif  // FLCE_PLAN_H
