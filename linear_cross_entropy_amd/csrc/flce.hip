// Fused linear cross-entropy forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// Computes, for H (N x D), W (V x D) and int32 targets y,
//     lse_i  = logsumexp_v (H W^T)[i, v],     loss_i = lse_i - (H W^T)[i, y_i]
// as defined on the page "A fused forward kernel for linear cross-entropy on
// Apple GPUs" (section 1), without ever storing the N x V logits.
//
// Two launches on the caller's stream:
//   1. flce_partials_kernel: a persistent-per-CU grid over (row block, vocab
//      chunk). Each workgroup owns BT tokens and a run of BV-row vocabulary
//      tiles. For every tile it contracts H_blk W_tile^T over the whole of D
//      on the matrix cores (bf16 x bf16 or fp32 x fp32 -> fp32), staging both
//      operands through LDS with direct buffer->LDS loads, then folds the
//      tile's logits, still in registers, into a running (max m, scaled sum
//      s) per token with the page's online update, and records the target
//      logit when the target index falls in the tile. At the end of its chunk
//      the workgroup writes one (m, s) per token.
//   2. flce_merge_kernel: per token, combines the chunks' (m, s) pairs with
//      the same update and writes lse = M + ln S and loss = lse - z_y.
//
// The update is applied per lane, not per row: every lane keeps its own
// (m, s) over the logits it holds, and lanes, waves and chunks are combined
// only at the end. This is the same identity the page uses between tiles
// (combining two partial states with the max-rescaled sum), applied to a
// different grouping of the vocabulary.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define FLCE_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_inff();

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
#define FLCE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00))

// Buffer resource word 3 for raw (unswizzled, stride 0) buffer accesses on
// gfx9-family parts: 32-bit data format, range checking against num_records.
constexpr int kRsrcWord3 = 0x00020000;
// Any offset at or above num_records reads as zero; every resource built here
// covers less than 2^31 bytes.
constexpr uint32_t kOutOfRange = 0x80000000u;

// ------------------------------------------------------------------ tiles
// One tile configuration: BV vocabulary rows x BT tokens per workgroup,
// WAVES_V x WAVES_T waves, each wave owning a (BV/WAVES_V) x (BT/WAVES_T)
// block of 32x32 MFMA tiles. K is staged 128 bytes (64 bf16 / 32 fp32) at a
// time, double-buffered in LDS.
constexpr int kBV = 256;
constexpr int kBT = 256;
constexpr int kWavesV = 2;
constexpr int kWavesT = 4;
constexpr int kThreads = 64 * kWavesV * kWavesT;
constexpr int kStageRowBytes = 128;
constexpr int kStageBytes = (kBV + kBT) * kStageRowBytes;
constexpr int kLdsBytes = 2 * kStageBytes;

struct PartialsArgs {
  const char* H;
  const char* W;
  const int32_t* y;
  float* part_m;      // [chunks][N]
  float* part_s;      // [chunks][N]
  float* z_target;    // [N]
  int N, V, row_bytes;
  int row_blocks, vocab_tiles, chunks;
  int xcd_rows, xcd_chunks;  // XCD group shape; xcd_rows == 0 disables the remap
};

// Element-type specific pieces: a 16-byte fragment and the matrix-core step
// that consumes one fragment of A and one of B (32x32 output, K = 16 bf16 or
// 4 x K = 2 fp32).
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 step(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  typedef f32x4 frag;
  static __device__ __forceinline__ f32x16 step(frag a, frag b, f32x16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row. gfx950's LDS
// serves a ds_read_b128 16 lanes (256 bytes, all 64 banks) at a time; lanes
// 0-15 of a fragment read rows r..r+15 at the same logical chunk, and
// (r >> 1) & 7 sends those 16 reads to 16 distinct 16-byte bank groups
// (rows r and r+1 differ in bank half, rows 2 apart in chunk). Measured on
// MI355X: ~247 B/clk/CU with this swizzle, ~127 with (r & 7), ~32 without.
__device__ __forceinline__ int swizzle(int row) { return (row >> 1) & 7; }

// Combine two partial states (m_a, s_a) and (m_b, s_b) of the online update:
// M = max(m_a, m_b), S = s_a e^(m_a - M) + s_b e^(m_b - M). A state with
// m = -inf is empty and contributes nothing.
__device__ __forceinline__ void combine(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float c = (M == kNegInf) ? 0.f : M * kLog2e;
  s = s * __builtin_amdgcn_exp2f(__builtin_fmaf(m, kLog2e, -c)) +
      s2 * __builtin_amdgcn_exp2f(__builtin_fmaf(m2, kLog2e, -c));
  m = M;
}

template <typename T>
__global__ __launch_bounds__(kThreads, 1) void flce_partials_kernel(PartialsArgs p) {
  typedef typename Mma<T>::frag Frag;
  constexpr int NW = kWavesV * kWavesT;
  constexpr int WV = kBV / kWavesV;          // vocabulary rows per wave
  constexpr int WT = kBT / kWavesT;          // tokens per wave
  constexpr int MB = WV / 32;                // 32x32 MFMA tiles along vocab
  constexpr int NB = WT / 32;                // ... and along tokens
  constexpr int ROWS_PER_WAVE = (kBV + kBT) / NW;  // LDS rows each wave fills per stage
  constexpr int LOADS = ROWS_PER_WAVE / 8;         // 16-byte loads per lane per stage
  static_assert(kBV % ROWS_PER_WAVE == 0, "a wave loads either W or H rows");
  static_assert(WV % 32 == 0 && WT % 32 == 0, "waves own whole MFMA tiles");

  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wv = wave % kWavesV;
  const int wt = wave / kWavesV;

  // ---- which (row block, chunk) this workgroup owns. Workgroups are handed
  // to the 8 XCDs round-robin by index; the remap gives each XCD a compact
  // xcd_rows x xcd_chunks block of the (row block, chunk) grid so that the
  // XCD's L2 sees few distinct H blocks and W tiles at a time.
  int rb, ch;
  {
    const int b = blockIdx.x;
    if (p.xcd_rows > 0) {
      const int x = b & 7, j = b >> 3;
      const int groups_c = p.chunks / p.xcd_chunks;
      rb = (x / groups_c) * p.xcd_rows + j / p.xcd_chunks;
      ch = (x % groups_c) * p.xcd_chunks + j % p.xcd_chunks;
    } else {
      rb = b / p.chunks;
      ch = b % p.chunks;
    }
  }
  const int t0 = rb * kBT;
  const int base_tiles = p.vocab_tiles / p.chunks;
  const int rem_tiles = p.vocab_tiles % p.chunks;
  const int tile_begin = ch * base_tiles + min(ch, rem_tiles);
  const int ntiles = base_tiles + (ch < rem_tiles ? 1 : 0);
  const int KS = (p.row_bytes + kStageRowBytes - 1) / kStageRowBytes;
  const int total = ntiles * KS;

  // ---- load plan: wave `wave` fills LDS rows [wave*ROWS_PER_WAVE, +ROWS_PER_WAVE)
  // of each stage; rows < kBV hold W (vocabulary) rows, the rest H (token) rows.
  // Lane l of load i writes LDS row r = row0 + 8*i + l/8, 16-byte slot l%8,
  // which holds the row's chunk (l%8) ^ swizzle(r).
  const int row0 = wave * ROWS_PER_WAVE;
  const bool w_wave = row0 < kBV;
  const int region_row0 = w_wave ? row0 : row0 - kBV;
  static_assert(ROWS_PER_WAVE % 16 == 0 && kBV % 16 == 0, "swizzle phase is set by 8*i + lane/8");
  // One buffer resource per operand for the whole chunk: the chunk's W rows
  // (the planner keeps them under 2^31 bytes) and the block's H rows. Rows
  // past V or N and bytes past D fall outside num_records and read as zero.
  const int v_chunk0 = tile_begin * kBV;
  const int region_rows = w_wave ? min(ntiles * kBV, p.V - v_chunk0) : min(kBT, p.N - t0);
  const char* region_base = w_wave ? p.W + (size_t)v_chunk0 * p.row_bytes : p.H + (size_t)t0 * p.row_bytes;
  const __amdgpu_buffer_rsrc_t ld_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)region_base, (short)0, region_rows * p.row_bytes, kRsrcWord3);
  int lane_row[LOADS], chunk_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    chunk_off[i] = ((lane & 7) ^ swizzle(8 * i + (lane >> 3))) * 16;
    lane_row[i] = region_row0 + 8 * i + (lane >> 3);
  }
  // Per tile: each load's byte offset at k = 0, or an out-of-range offset for
  // rows past the region (an out-of-range base stays out of range after
  // adding k offsets below 2^31).
  uint32_t tile_off[LOADS];
  auto set_tile = [&](int tile) {
    const int first = w_wave ? tile * kBV : 0;  // H rows stay put across tiles
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = first + lane_row[i];
      tile_off[i] = r < region_rows ? (uint32_t)(r * p.row_bytes + chunk_off[i]) : kOutOfRange;
    }
  };

  int issue_tile = 0, issue_ks = 0;
  set_tile(0);
  auto issue = [&](int buf) {
    const int kbyte = issue_ks * kStageRowBytes;
    FLCE_LDS char* dst = (FLCE_LDS char*)(smem) + buf * kStageBytes + row0 * kStageRowBytes;
    if (kbyte + kStageRowBytes <= p.row_bytes) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_rsrc, (FLCE_LDS void*)(dst + i * 8 * kStageRowBytes), 16,
                                                 tile_off[i] + kbyte, 0, 0, 0);
    } else {
      // last, partial k-stage: chunks past the end of the row read as zero
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t off = kbyte + chunk_off[i] < p.row_bytes ? tile_off[i] + kbyte : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_rsrc, (FLCE_LDS void*)(dst + i * 8 * kStageRowBytes), 16,
                                                 off, 0, 0, 0);
      }
    }
    if (++issue_ks == KS) {
      issue_ks = 0;
      set_tile(++issue_tile);
    }
  };

  // ---- fragment addresses: a 32x32xK MFMA tile reads, per lane, row
  // (lane % 32) of its 32-row block and 16-byte chunk 2*kb + lane/32.
  int koff[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    koff[kb] = (lane & 31) * kStageRowBytes + (((2 * kb + (lane >> 5)) ^ swizzle(lane & 31)) * 16);
  const int a_row = wv * WV;
  const int b_row = kBV + wt * WT;

  // ---- per-lane online state for the NB token columns this lane holds.
  // 32x32 MFMA output layout: lane l holds column l%32 and, in register r,
  // row 8*(r/4) + 4*(l/32) + r%4 of the 32x32 tile.
  float m_run[NB], s_run[NB], zt[NB];
  bool zhit[NB];
  int ytok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    s_run[nb] = 0.f;
    zt[nb] = 0.f;
    zhit[nb] = false;
    const int tok = t0 + wt * WT + nb * 32 + (lane & 31);
    ytok[nb] = tok < p.N ? p.y[tok] : -1;
  }

  f32x16 acc[MB][NB];
  Frag fa[2][MB], fb[2][NB];  // two fragment sets: one being consumed, one in flight

  auto read_frags = [&](int set, const char* sb, int kb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      fa[set][mb] = *(const Frag*)(sb + (a_row + mb * 32) * kStageRowBytes + koff[kb]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      fb[set][nb] = *(const Frag*)(sb + (b_row + nb * 32) * kStageRowBytes + koff[kb]);
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Mma<T>::step(fa[set][mb], fb[set][nb], acc[mb][nb]);
  };
  constexpr int MFMA_PER_KB = MB * NB * (sizeof(T) == 2 ? 1 : 4);  // matrix instructions per k-block

  // ---- main loop over the chunk's stages (tile-major, k-stage minor); stage g
  // lives in LDS buffer g & 1. After the barrier that publishes stage g (and
  // retires stage g - 1), a wave reads its first fragments of stage g, issues
  // the loads of stage g + 1 into the retired buffer, then runs the stage's
  // four k-blocks with the next k-block's fragment reads spread between the
  // current k-block's MFMAs.
  issue(0);
  int ks = 0, tile = 0;
  for (int g = 0; g < total; ++g) {
    FLCE_WAIT_VMCNT(0);          // this wave's loads of stage g have landed in LDS
    __syncthreads();             // ... and everyone's; stage g - 1's buffer is free
    const char* sb = smem + (g & 1) * kStageBytes;
    read_frags(0, sb, 0);
    if (g + 1 < total) issue((g + 1) & 1);
    if (ks == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb + 1 < 4) read_frags((kb + 1) & 1, sb, kb + 1);
      mfmas(kb & 1);
    }
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
#pragma unroll
      for (int j = 0; j < MB + NB; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MFMA_PER_KB - (MB + NB), 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MFMA_PER_KB, 0);
    if (++ks < KS) continue;
    ks = 0;

    // ---- epilogue of one vocabulary tile, entirely in registers
    const int vw = (tile_begin + tile) * kBV + a_row;   // first vocabulary row of this wave
    ++tile;
    if (vw + WV > p.V) {
      // ragged last tile: vocabulary rows >= V are not logits at all
      int lim = p.V - vw - 4 * (lane >> 5);
      asm volatile("" : "+v"(lim));  // compared here, not hoisted as per-register lane masks
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mb * 32 + 8 * (r >> 2) + (r & 3) >= lim) acc[mb][nb][r] = kNegInf;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // target logit: kept by the one lane holding (y, token); written at the end of the chunk
      const int rel = ytok[nb] - vw;
      if ((unsigned)rel < (unsigned)WV && ((rel >> 2) & 1) == (lane >> 5)) {
        int want = rel;
        asm volatile("" : "+v"(want));  // likewise
        const int want_mb = want >> 5;
        const int want_r = ((want & 31) >> 3) * 4 + (want & 3);
        float val = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mb == want_mb && r == want_r) val = acc[mb][nb][r];
        zt[nb] = val;
        zhit[nb] = true;
      }
      // online update: m' = max(m, m_tile), s' = s e^(m - m') + sum_j e^(z_j - m')
      float tmax = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc[mb][nb][r]);
      const float m_new = fmaxf(m_run[nb], tmax);
      const float c = (m_new == kNegInf) ? 0.f : m_new * kLog2e;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][r], kLog2e, -c));
          s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][r + 1], kLog2e, -c));
        }
      s_run[nb] = s_run[nb] * __builtin_amdgcn_exp2f(__builtin_fmaf(m_run[nb], kLog2e, -c)) + (s0 + s1);
      m_run[nb] = m_new;
    }
  }

  // ---- target logits found in this chunk
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    if (zhit[nb]) p.z_target[t0 + wt * WT + nb * 32 + (lane & 31)] = zt[nb];

  // ---- end of chunk: combine the two half-waves, then the kWavesV waves that
  // share a token range, in a fixed order (deterministic), and write one
  // (m, s) per token.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float m2 = __shfl_xor(m_run[nb], 32);
    const float s2 = __shfl_xor(s_run[nb], 32);
    combine(m_run[nb], s_run[nb], m2, s2);
  }
  __syncthreads();  // every wave is done with the stage buffers
  float* red = (float*)smem;  // [kWavesV][kBT] m, then [kWavesV][kBT] s
  if (lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wt * WT + nb * 32 + lane;
      red[wv * kBT + col] = m_run[nb];
      red[(kWavesV + wv) * kBT + col] = s_run[nb];
    }
  }
  __syncthreads();
  if (wv == 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wt * WT + nb * 32 + lane;
      float m = red[col], s = red[kWavesV * kBT + col];
#pragma unroll
      for (int w = 1; w < kWavesV; ++w) combine(m, s, red[w * kBT + col], red[(kWavesV + w) * kBT + col]);
      const int tok = t0 + col;
      if (tok < p.N) {
        p.part_m[(size_t)ch * p.N + tok] = m;
        p.part_s[(size_t)ch * p.N + tok] = s;
      }
    }
  }
}

// Merge: one thread per token. M = max_c m_c, S = sum_c s_c e^(m_c - M),
// lse = M + ln S, loss = lse - z_y (NaN when y is not in [0, V)).
__global__ __launch_bounds__(256) void flce_merge_kernel(const float* __restrict__ part_m,
                                                         const float* __restrict__ part_s,
                                                         const float* __restrict__ z_target,
                                                         const int32_t* __restrict__ y, int N, int V,
                                                         int chunks, float* __restrict__ loss,
                                                         float* __restrict__ lse) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  float M = kNegInf;
  for (int c = 0; c < chunks; ++c) M = fmaxf(M, part_m[(size_t)c * N + i]);
  float S = 0.f;
  for (int c = 0; c < chunks; ++c) {
    const float m = part_m[(size_t)c * N + i];
    const float w = (m == kNegInf) ? 0.f : expf(m - M);
    S += part_s[(size_t)c * N + i] * w;
  }
  const float l = M + logf(S);
  if (lse) lse[i] = l;
  const int t = y[i];
  loss[i] = (t >= 0 && t < V) ? l - z_target[i] : __builtin_nanf("");
}

// ------------------------------------------------------------------ host side
constexpr int kSlots = 256;       // workgroups resident at once: one per CU
constexpr size_t kAlign = 256;

struct Plan {
  int N, V, row_bytes, dtype;
  int row_blocks, vocab_tiles, chunks, grid, xcd_rows, xcd_chunks;
  size_t off_m, off_s, off_z, ws_bytes;
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int make_plan(int64_t N, int64_t D, int64_t V, int dtype, Plan* pl) {
  if (dtype != FLCE_BF16 && dtype != FLCE_FP32) return FLCE_ERR_UNSUPPORTED;
  if (N < 0 || D < 1 || V < 1) return FLCE_ERR_INVALID_ARG;
  const int64_t es = dtype == FLCE_BF16 ? 2 : 4;
  const int64_t rb = D * es;
  if (rb % 16 != 0) return FLCE_ERR_UNSUPPORTED;
  // 32-bit offsets inside one tile's buffer resource, int32 indices elsewhere
  if ((int64_t)kBV * rb >= (int64_t(1) << 31) || N > INT32_MAX / 2 || V > INT32_MAX - kBV)
    return FLCE_ERR_UNSUPPORTED;
  pl->N = (int)N;
  pl->V = (int)V;
  pl->row_bytes = (int)rb;
  pl->dtype = dtype;
  pl->row_blocks = (int)((N + kBT - 1) / kBT);
  pl->vocab_tiles = (int)((V + kBV - 1) / kBV);
  // chunks per row block: minimise the makespan in tile-times,
  // ceil(row_blocks*c / slots) * ceil(vocab_tiles / c); ties go to fewer chunks.
  int best_c = 0;
  int64_t best_cost = INT64_MAX;
  const int RB = pl->row_blocks > 0 ? pl->row_blocks : 1;
  for (int c = 1; c <= pl->vocab_tiles; ++c) {
    const int64_t rounds = ((int64_t)RB * c + kSlots - 1) / kSlots;
    const int64_t per = (pl->vocab_tiles + c - 1) / c;
    if (per * kBV * rb >= (int64_t(1) << 31)) continue;  // one buffer resource per chunk
    const int64_t cost = rounds * per;
    if (cost < best_cost) {
      best_cost = cost;
      best_c = c;
    }
  }
  if (best_c == 0) return FLCE_ERR_UNSUPPORTED;
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

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_inputs(const void* H, const void* W, const int32_t* y, int64_t N) {
  if (N == 0) return FLCE_OK;
  if (!H || !W || !y) return FLCE_ERR_INVALID_ARG;
  if (!aligned(H, 16) || !aligned(W, 16) || !aligned(y, 4)) return FLCE_ERR_INVALID_ARG;
  return FLCE_OK;
}

int check_workspace(const Plan& pl, const void* ws, size_t bytes) {
  if (!ws || bytes < pl.ws_bytes || !aligned(ws, kAlign)) return FLCE_ERR_INVALID_ARG;
  return FLCE_OK;
}

int launch_partials(const Plan& pl, const void* H, const void* W, const int32_t* y, void* ws,
                    hipStream_t stream) {
  PartialsArgs a;
  a.H = (const char*)H;
  a.W = (const char*)W;
  a.y = y;
  a.part_m = (float*)((char*)ws + pl.off_m);
  a.part_s = (float*)((char*)ws + pl.off_s);
  a.z_target = (float*)((char*)ws + pl.off_z);
  a.N = pl.N;
  a.V = pl.V;
  a.row_bytes = pl.row_bytes;
  a.row_blocks = pl.row_blocks;
  a.vocab_tiles = pl.vocab_tiles;
  a.chunks = pl.chunks;
  a.xcd_rows = pl.xcd_rows;
  a.xcd_chunks = pl.xcd_chunks;
  if (pl.dtype == FLCE_BF16)
    hipLaunchKernelGGL(flce_partials_kernel<__bf16>, dim3(pl.grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(flce_partials_kernel<float>, dim3(pl.grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int launch_merge(const Plan& pl, const int32_t* y, float* loss, float* lse, const void* ws,
                 hipStream_t stream) {
  const float* m = (const float*)((const char*)ws + pl.off_m);
  const float* s = (const float*)((const char*)ws + pl.off_s);
  const float* z = (const float*)((const char*)ws + pl.off_z);
  hipLaunchKernelGGL(flce_merge_kernel, dim3((pl.N + 255) / 256), dim3(256), 0, stream, m, s, z, y,
                     pl.N, pl.V, pl.chunks, loss, lse);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

}  // namespace

extern "C" {

int flce_version(void) { return 100; }

const char* flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_INVALID_ARG: return "invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case FLCE_ERR_HIP: return "HIP runtime error";
    case FLCE_ERR_OOM: return "workspace allocation failed";
    default: return "unknown status";
  }
}

int flce_get_plan(int64_t N, int64_t D, int64_t V, int dtype, flce_plan_t* out) {
  if (!out) return FLCE_ERR_INVALID_ARG;
  Plan pl;
  const int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return rc;
  out->tile_vocab = kBV;
  out->tile_tokens = kBT;
  out->row_blocks = pl.row_blocks;
  out->vocab_tiles = pl.vocab_tiles;
  out->chunks = pl.chunks;
  out->grid = N > 0 ? pl.grid : 0;
  out->xcd_rows = pl.xcd_rows;
  out->xcd_chunks = pl.xcd_chunks;
  out->threads = kThreads;
  out->lds_bytes = kLdsBytes;
  out->workspace_bytes = N > 0 ? pl.ws_bytes : 0;
  return FLCE_OK;
}

size_t flce_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype) {
  Plan pl;
  if (make_plan(N, D, V, dtype, &pl) != FLCE_OK || N == 0) return 0;
  return pl.ws_bytes;
}

int flce_partials(const void* H, const void* W, const int32_t* targets, int64_t N, int64_t D,
                  int64_t V, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return rc;
  if ((rc = check_inputs(H, W, targets, N)) != FLCE_OK) return rc;
  if (N == 0) return FLCE_OK;
  if ((rc = check_workspace(pl, workspace, workspace_bytes)) != FLCE_OK) return rc;
  return launch_partials(pl, H, W, targets, workspace, (hipStream_t)stream);
}

int flce_merge(const int32_t* targets, int64_t N, int64_t D, int64_t V, int dtype, float* loss_out,
               float* lse_out, const void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return rc;
  if (N == 0) return FLCE_OK;
  if (!targets || !loss_out || !aligned(targets, 4) || !aligned(loss_out, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return FLCE_ERR_INVALID_ARG;
  if ((rc = check_workspace(pl, workspace, workspace_bytes)) != FLCE_OK) return rc;
  return launch_merge(pl, targets, loss_out, lse_out, workspace, (hipStream_t)stream);
}

int flce_forward_ws(const void* H, const void* W, const int32_t* targets, int64_t N, int64_t D,
                    int64_t V, int dtype, float* loss_out, float* lse_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return rc;
  if ((rc = check_inputs(H, W, targets, N)) != FLCE_OK) return rc;
  if (N == 0) return FLCE_OK;
  if (!loss_out || !aligned(loss_out, 4) || (lse_out && !aligned(lse_out, 4)))
    return FLCE_ERR_INVALID_ARG;
  if ((rc = check_workspace(pl, workspace, workspace_bytes)) != FLCE_OK) return rc;
  if ((rc = launch_partials(pl, H, W, targets, workspace, (hipStream_t)stream)) != FLCE_OK) return rc;
  return launch_merge(pl, targets, loss_out, lse_out, workspace, (hipStream_t)stream);
}

int flce_forward(const void* H, const void* W, const int32_t* targets, int64_t N, int64_t D,
                 int64_t V, int dtype, float* loss_out, float* lse_out, void* stream) {
  Plan pl;
  int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return rc;
  if ((rc = check_inputs(H, W, targets, N)) != FLCE_OK) return rc;
  if (N == 0) return FLCE_OK;
  if (!loss_out || !aligned(loss_out, 4) || (lse_out && !aligned(lse_out, 4)))
    return FLCE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, pl.ws_bytes, s) != hipSuccess || !ws) {
    (void)hipGetLastError();
    return FLCE_ERR_OOM;
  }
  rc = launch_partials(pl, H, W, targets, ws, s);
  if (rc == FLCE_OK) rc = launch_merge(pl, targets, loss_out, lse_out, ws, s);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == FLCE_OK) rc = FLCE_ERR_HIP;
  return rc;
}

}  // extern "C"
