// Fused linear cross-entropy, forward and backward, for AMD Instinct MI355X
// (gfx950, CDNA4).
//
// Forward: for H (N x D), W (V x D) and int32 targets y,
//     lse_i  = logsumexp_v (H W^T)[i, v],     loss_i = lse_i - (H W^T)[i, y_i]
// as defined on the page "Een gefuseerde forward-kernel voor lineaire
// cross-entropy op Apple-GPU's" (section 1), without ever storing the N x V
// logits. Two launches on the caller's stream:
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
//
// Backward (gradients of sum_i g_i loss_i; the page's training path keeps
// the forward's lse and regenerates the logits, section 1): the same tile
// loop recomputes Z and writes dZ = g (softmax - onehot) (flce_dz_kernel),
// and runs the two products dW = dZ^T H with a store epilogue
// (flce_gemm_kernel) on K-contiguous transposed copies (flce_transpose_kernel)
// and dH = dZ W, for bf16 reading dZ from its transposed copy through
// transposing LDS reads (flce_gemmt_kernel); when that product's tiles would
// leave compute units idle, its contraction over the vocabulary is split
// into float32 partial sums that flce_ksum_kernel adds in a fixed order.
//
// Quantised head (the page's first prototype handled quantised output heads,
// section 2; the format here is a reading, stated in flce.h): the vocabulary
// runs in slices, each dequantised to bf16 by flce_dequant_kernel into the
// workspace and run through the unchanged partials kernel with its targets
// offset by the slice's first row; one merge covers all slices' chunks.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "flce.h"
#include "flce_plan.h"

namespace {

using namespace flce_plan;

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

// What the tile loop does with each finished tile of Z = A B^T (A: the rows
// along the tile's vocabulary axis, B: the rows along its token axis).
enum TileMode {
  kForward = 0,  // online (max, sum) per token, target capture, per-chunk partials
  kDz = 1,       // dZ = g (softmax - onehot), written transposed (and row-major if dz is set)
  kGemm = 2,     // plain C[a][b] = Z
  kGemmT = 3,    // C[b][a] = Z with B read from a [k][b] matrix (bf16 only)
};

struct TileArgs {
  const char* H;      // B operand: b_rows x K (tokens in the forward)
  const char* W;      // A operand: a_rows x K (vocabulary rows in the forward)
  int N, V, row_bytes;  // b_rows, a_rows, K in bytes (both operands' row length)
  int row_blocks, vocab_tiles, chunks;
  int xcd_rows, xcd_chunks;  // XCD group shape; xcd_rows == 0 disables the remap
  // kForward and kDz
  const int32_t* y;   // [N] targets
  int v_off;          // vocabulary index of W's first row: a target y counts as row y - v_off
  // kForward
  float* part_m;      // [chunks][N]
  float* part_s;      // [chunks][N]
  float* z_target;    // [N]
  // kDz: lse and upstream gradient per token; dZ as [v][dzt_ld] and, when dz is
  // not null, also as [tok][dz_ld]
  const float* lse;
  const float* grad;
  char* dz;
  char* dzt;
  int dz_ld, dzt_ld;  // row lengths in elements (>= the valid extents; the rest is written as 0)
  int dz_rows;        // tokens to write in dz / columns in dzt (N rounded up)
  int dz_cols;        // vocabulary rows to write (V rounded up)
  // kGemm: C[a][b] at C[a * ldc + b]; kGemmT: C[b][a] at C[b * ldc + a]
  float* C;           // fp32
  int ldc;
  // kGemmT: B is stored transposed, B[b][k] at H[k * ldb + b] (elements); K = row_bytes / 2
  int ldb;
  // kGemmT split over K: the grid is ksplit copies of the row_blocks x chunks
  // grid, copy s contracting k-stages [s * ks_per, (s + 1) * ks_per) and
  // writing its partial C to C + s * N * ldc
  int ksplit, ks_per;
  // kGemm and kGemmT: add Z to C instead of overwriting it
  int accumulate;
};

// Element-type and MFMA-shape specific pieces: a 16-byte fragment, the
// accumulator of one M x M output tile, and the matrix-core step that
// consumes one fragment of A and one of B (bf16: 32x32 outputs with K = 16,
// or 16x16 outputs with K = 32; fp32: 32x32 outputs as 4 x K = 2).
template <typename T, int M> struct Mma;

template <> struct Mma<__bf16, 32> {
  typedef bf16x8 frag;
  typedef f32x16 acc;
  static __device__ __forceinline__ acc step(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<__bf16, 16> {
  typedef bf16x8 frag;
  typedef f32x4 acc;
  static __device__ __forceinline__ acc step(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float, 32> {
  typedef f32x4 frag;
  typedef f32x16 acc;
  static __device__ __forceinline__ acc step(frag a, frag b, acc c) {
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

// XOR swizzle of the 32 16-byte chunks of a k-row of a transposed B stage
// (kGemmT). In a transposing fragment read each half-wave takes the same 64
// bytes (4 chunks, starting at a multiple of 4) from each of 4 consecutive
// k-rows, and the rows are 512 bytes apart, i.e. on the same banks. XOR-ing
// k-row k's chunk index with 4 (k & 3) moves the four pieces to the four
// different 64-byte quarters of the 256 bytes the 64 banks cover.
__device__ __forceinline__ int bswizzle(int krow) { return (krow & 3) * 4; }

// Online-update state (m, s) in base 2: m is the running maximum logit and
// s = sum_j 2^(z_j log2(e) - off(m)) with off(m) = fl(m * log2(e)), the fp32
// product, so that e^lse = 2^off(m) * s. Every rescale multiplies by
// 2^(off(m_old) - off(m_new)), the difference of the same rounded offsets the
// terms were taken against: an unchanged maximum rescales by exactly 1, and
// rounding does not compound over the hundreds of tiles a state absorbs.
// The library is built with -ffp-contract=off (every FMA in this file is an
// explicit __builtin_fmaf): contracting off2(m_old) - c back into
// fma(m_old, log2 e, -c) would bring the rounding residual back into every
// rescale, an error that compounds over the tiles (measured: 1.9e-3 in lse at
// |lse| = 366 with D = 8192, against 4.6e-4 without it).
__device__ __forceinline__ float off2(float m) { return m * kLog2e; }

// Combine two partial states (m_a, s_a) and (m_b, s_b) of the online update:
// M = max(m_a, m_b), S = s_a e^(m_a - M) + s_b e^(m_b - M). A state with
// m = -inf is empty (s = 0) and contributes nothing.
__device__ __forceinline__ void combine(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float c = (M == kNegInf) ? 0.f : off2(M);
  s = s * __builtin_amdgcn_exp2f(off2(m) - c) + s2 * __builtin_amdgcn_exp2f(off2(m2) - c);
  m = M;
}

// Four consecutive elements to (8- or 16-byte aligned) global memory.
__device__ __forceinline__ void store4(char* dst, const __bf16 (&q)[4]) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = {q[0], q[1], q[2], q[3]};
  *(bf16x4*)dst = v;
}
__device__ __forceinline__ void store4(char* dst, const float (&q)[4]) {
  const f32x4 v = {q[0], q[1], q[2], q[3]};
  *(f32x4*)dst = v;
}

// The tile loop shared by the forward, the backward's dZ pass and the
// backward's products: one workgroup owns a block of kBT B rows and a chunk of
// kBV-row A tiles, contracts each tile over the whole of K on the matrix cores
// and hands the finished tile, in registers, to the MODE's epilogue.
template <typename T, typename C, int MODE>
__device__ __forceinline__ void tile_loop(const TileArgs& p) {
  typedef Mma<T, C::M> MmaT;
  typedef typename MmaT::frag Frag;
  typedef typename MmaT::acc Acc;
  constexpr int kBV = C::BV, kBT = C::BT, kWavesV = C::WAVES_V;
  constexpr int WV = C::WV, WT = C::WT, MB = C::MB, NB = C::NB;
  // MFMA shape: M x M output tiles, KSTEPS instructions' K per 128-byte stage,
  // ACC accumulator registers per lane and tile, KCH 16-byte chunks of a row
  // per K step. Output layout of an M x M tile: lane l holds column l % M;
  // register r holds row lane_row + row_in(r), lane_row = 4 (l / M) for both
  // shapes (32x32: row_in(r) = 8 (r / 4) + r % 4; 16x16: row_in(r) = r).
  constexpr int M = C::M, KSTEPS = C::KSTEPS, ACC = C::ACC, KCH = 64 / M;
  static_assert(M == 32 || sizeof(T) == 2, "fp32 runs the 32x32 shape");
  constexpr Acc kZeroAcc = {};
  constexpr int WLOADS = C::WLOADS, HLOADS = C::HLOADS;
  constexpr int kStageBytes = C::STAGE_BYTES;

  // The forward on 16x16 tiles keeps the workgroup's targets in LDS beside the
  // stages (kBT ints) instead of in registers: a lane holds four token
  // columns there, and the registers are needed for the accumulators and
  // fragments (held in registers, the targets were spilled and reloaded every
  // tile, each reload waiting for the next stage's loads as well).
  // The running maxima go there too (one float per lane and token column),
  // when they fit: held across the stage loop but used only once per tile,
  // they were the other values spilled.
  constexpr bool kYLds = MODE == kForward && M == 16 && C::LDS_BYTES + kBT * 4 <= 160 * 1024;
  constexpr int kMLdsBytes = C::NW * NB * 64 * 4;
  constexpr bool kMLds = kYLds && C::LDS_BYTES + kBT * 4 + kMLdsBytes <= 160 * 1024;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES + (kYLds ? kBT * 4 : 0) + (kMLds ? kMLdsBytes : 0)];

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
    const int b = MODE == kGemmT ? (int)blockIdx.x % (p.row_blocks * p.chunks) : (int)blockIdx.x;
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
  const int KS_all = (p.row_bytes + kStageRowBytes - 1) / kStageRowBytes;
  int kslice = 0, kfirst = 0, KS = KS_all;  // this workgroup's k-stages: [kfirst, kfirst + KS)
  if constexpr (MODE == kGemmT) {
    kslice = (int)blockIdx.x / (p.row_blocks * p.chunks);
    kfirst = kslice * p.ks_per;
    KS = min(p.ks_per, KS_all - kfirst);
  }
  const int total = ntiles * KS;

  // ---- load plan. Each stage holds kBV W rows (LDS rows [0, kBV)) and kBT H
  // rows (LDS rows [kBV, kBV + kBT)), 128 bytes of K each. Wave w fills W rows
  // [w*WROWS, +WROWS) and H rows [w*HROWS, +HROWS). Lane l of a load covering
  // LDS rows r0..r0+7 writes row r0 + l/8, 16-byte slot l%8, which holds the
  // row's chunk (l%8) ^ swizzle(row).
  //
  // One buffer resource per operand for the whole chunk: the chunk's W rows
  // (the planner keeps them under 2^31 bytes) and the block's H rows. Rows
  // past V or N and bytes past D fall outside num_records and read as zero.
  const int v_chunk0 = tile_begin * kBV;
  const int w_rows = min(ntiles * kBV, p.V - v_chunk0);
  const int h_rows = min(kBT, p.N - t0);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W + (size_t)v_chunk0 * p.row_bytes), (short)0, w_rows * p.row_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t h_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.H + (size_t)t0 * p.row_bytes), (short)0, h_rows * p.row_bytes, kRsrcWord3);
  const int w_row0 = wave * C::WROWS;        // first W row (within the tile) this wave fills
  const int h_row0 = wave * C::HROWS;        // first H row this wave fills
  int w_chunk[WLOADS], h_chunk[HLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) w_chunk[i] = ((lane & 7) ^ swizzle(w_row0 + 8 * i + (lane >> 3))) * 16;
#pragma unroll
  for (int i = 0; i < HLOADS; ++i) h_chunk[i] = ((lane & 7) ^ swizzle(kBV + h_row0 + 8 * i + (lane >> 3))) * 16;
  // Byte offset of each load at k = 0 (W: in the chunk's first tile), or an
  // out-of-range offset for rows past the region (an out-of-range base stays
  // out of range after adding k < 2^31).
  uint32_t w_off[WLOADS], h_off[HLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) {
    const int r = w_row0 + 8 * i + (lane >> 3);
    w_off[i] = r < w_rows ? (uint32_t)(r * p.row_bytes + w_chunk[i]) : kOutOfRange;
  }
#pragma unroll
  for (int i = 0; i < HLOADS; ++i) {
    const int r = h_row0 + 8 * i + (lane >> 3);
    h_off[i] = r < h_rows ? (uint32_t)(r * p.row_bytes + h_chunk[i]) : kOutOfRange;
  }
  // kGemmT: the B part of a stage holds 64 k-rows of kBT columns (kBT * 2
  // bytes each) of the transposed B, in the same LDS bytes. Load j of wave w
  // fills k-rows 2 (w * HLOADS + j) and the next one: lane l writes 16-byte
  // slot l % 32 of k-row 2 (w * HLOADS + j) + l / 32, which holds that row's
  // chunk (l % 32) ^ bswizzle(row). The offsets are relative to a buffer
  // resource based at the stage's first k-row (and this block's first column),
  // made per stage: k-rows past K fall outside it and read as zero.
  constexpr int kBRowBytes = kBT * 2;
  if constexpr (MODE == kGemmT) {
    static_assert(sizeof(T) == 2 && 64 * kBRowBytes == kBT * kStageRowBytes, "transposed B: bf16, 64 k-rows a stage");
    static_assert(M == 32, "transposed B: 32x32 fragments");
#pragma unroll
    for (int i = 0; i < HLOADS; ++i) {
      const int krow = 2 * (wave * HLOADS + i) + (lane >> 5);
      h_off[i] = (uint32_t)(krow * p.ldb * 2 + (((lane & 31) ^ bswizzle(krow)) * 16));
    }
  }

  // On the last k-stage of a row that is not a multiple of 128 bytes long,
  // only lanes whose chunk starts inside the row may load: bit i of tail_ok
  // (W loads, then H loads) says whether load i's chunk does.
  constexpr int NLOADS = WLOADS + HLOADS;
  const int tail_bytes = p.row_bytes - (KS_all - 1) * kStageRowBytes;
  uint32_t tail_ok = 0;
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) tail_ok |= (w_chunk[i] < tail_bytes ? 1u : 0u) << i;
#pragma unroll
  for (int i = 0; i < HLOADS; ++i) tail_ok |= (h_chunk[i] < tail_bytes ? 1u : 0u) << (WLOADS + i);

  int issue_tile = 0, issue_ks = 0;
  // kGemmT: the resource for the transposed B of the stage being issued
  auto b_stage_rsrc = [&](int ks) {
    const int k0 = ks * 64;
    const int krows = min(64, p.row_bytes / 2 - k0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(p.H + ((size_t)k0 * p.ldb + t0) * 2), (short)0,
                                             max(krows * p.ldb - t0, 0) * 2, kRsrcWord3);
  };
  __amdgpu_buffer_rsrc_t bt_rsrc = b_stage_rsrc(kfirst);
  // Load i (W loads first) of the next stage into LDS buffer buf. With
  // live == false the load reads out of range: it fills the buffer with
  // zeros and touches no memory. (offsets are cast explicitly: without it the
  // host-side instantiation of this template drops the kernel's launch stub)
  auto issue_one = [&](int buf, int i, bool live) {
    const int kbyte = (kfirst + issue_ks) * kStageRowBytes;
    const bool whole = kbyte + kStageRowBytes <= p.row_bytes;
    const bool ok = live && (whole || ((tail_ok >> i) & 1u));
    FLCE_LDS char* sbuf = (FLCE_LDS char*)(smem) + buf * kStageBytes;
    if (i < WLOADS) {
      const uint32_t off = ok ? w_off[i] + kbyte : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rsrc, (FLCE_LDS void*)(sbuf + (w_row0 + 8 * i) * kStageRowBytes), 16, off, 0, 0, 0);
    } else if constexpr (MODE == kGemmT) {
      const int j = i - WLOADS;
      const uint32_t off = live ? h_off[j] : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          bt_rsrc, (FLCE_LDS void*)(sbuf + (kBV + h_row0 + 8 * j) * kStageRowBytes), 16, off, 0, 0, 0);
    } else {
      const int j = i - WLOADS;
      const uint32_t off = ok ? h_off[j] + kbyte : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          h_rsrc, (FLCE_LDS void*)(sbuf + (kBV + h_row0 + 8 * j) * kStageRowBytes), 16, off, 0, 0, 0);
    }
  };
  // Moving to the next tile moves every W row by kBV rows: a load whose row
  // is still inside the chunk advances by kBV rows' bytes, one past it reads
  // out of range from then on. Only the lane's row within its 8-row load
  // group varies per lane, and it is recomputed here rather than kept live.
  auto issue_done = [&]() {
    if constexpr (MODE == kGemmT) bt_rsrc = b_stage_rsrc(kfirst + (issue_ks + 1 == KS ? 0 : issue_ks + 1));
    if (++issue_ks == KS) {
      issue_ks = 0;
      ++issue_tile;
      int l8 = threadIdx.x & 63;
      asm volatile("" : "+v"(l8));
      l8 >>= 3;
      const uint32_t step = (uint32_t)(kBV * p.row_bytes);
#pragma unroll
      for (int i = 0; i < WLOADS; ++i) {
        const int lim = w_rows - issue_tile * kBV - w_row0 - 8 * i;  // rows of load i still inside the chunk
        w_off[i] = l8 < lim ? w_off[i] + step : kOutOfRange;
      }
    }
  };

  // ---- fragment addresses: an M x M MFMA tile's operand fragment for K step
  // kb is, per lane, row (lane % M) of its M-row block and 16-byte chunk
  // KCH*kb + lane/M of the stage row (32x32: 2 kb + lane/32; 16x16: 4 kb + lane/16).
  int koff[KSTEPS];
#pragma unroll
  for (int kb = 0; kb < KSTEPS; ++kb)
    koff[kb] = (lane % M) * kStageRowBytes + (((KCH * kb + lane / M) ^ swizzle(lane % M)) * 16);
  const int a_row = wv * WV;
  const int b_row = kBV + wt * WT;

  // ---- per-lane online state for the NB token columns this lane holds
  // (column l % M of each M x M tile; see the output layout above).
  const int lane_row = 4 * (lane / M);
  auto row_in = [](int r) { return M == 32 ? 8 * (r >> 2) + (r & 3) : r; };
  float m_run[NB], s_run[NB];  // m_run unused with kMLds
  int ytok[NB];  // unused with kYLds
  float* msm = (float*)(smem + C::LDS_BYTES + kBT * 4) + wave * NB * 64 + lane;  // kMLds: running max of column nb at [nb * 64]
  float l2tok[NB], gtok[NB];  // kDz: lse * log2(e) and the upstream gradient of each token
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    if constexpr (kMLds) msm[nb * 64] = kNegInf;  // read only after the prologue's barrier
    s_run[nb] = 0.f;
    const int tok = t0 + wt * WT + nb * M + (lane % M);
    ytok[nb] = -1;
    l2tok[nb] = 0.f;
    gtok[nb] = 0.f;
    if constexpr ((MODE == kForward && !kYLds) || MODE == kDz) {
      if (tok < p.N) ytok[nb] = p.y[tok] - p.v_off;
    }
    if constexpr (MODE == kDz) {
      if (tok < p.N) {
        l2tok[nb] = p.lse[tok] * kLog2e;
        gtok[nb] = p.grad[tok];
      }
    }
  }

  Acc acc[MB][NB];
  // Fragments: the NB H fragments of the current k-block and of the next one
  // (two sets), and a rolling window of kASlots W fragments. W fragment q of
  // a stage (q = kb*MB + mb) lives in slot q % kASlots; once the MFMAs that
  // use it have issued, the slot receives fragment q + kASlots, and across
  // the stage boundary fragment j of the next stage (QN is a multiple of
  // kASlots, so that is slot j again).
  constexpr int QN = KSTEPS * MB;  // W fragments per stage
  constexpr int kASlots = QN % 3 == 0 ? 3 : 4;
  static_assert(QN % kASlots == 0 && MB >= kASlots, "rolling window");
  // kGemmT keeps all four k-blocks' B fragments of a stage (see the main loop)
  constexpr bool kTB = MODE == kGemmT;
  constexpr int kBSets = kTB ? 4 : 2;
  Frag fa[kASlots], fb[kBSets][NB];
  auto read_a = [&](const char* sb, int q) {
    fa[q % kASlots] = *(const Frag*)(sb + (a_row + (q % MB) * M) * kStageRowBytes + koff[q / MB]);
  };
  // kGemmT: a B fragment (column n = lane % 32, k = 8 (lane / 32) + 0..7) is
  // two transposing reads of 4 k each. Within a 16-lane group, lane s names
  // k-row k0 + s / 4 and columns n0 + 4 (s % 4) .. + 3, and lane s receives
  // column n0 + s of k-rows k0 .. k0 + 3; boff[nb][h] is that address for the
  // lane (k0 = 8 (lane / 32) + 4h at k-block 0, n0 = 16 ((lane / 16) % 2)).
  int boff[NB][2];
  if constexpr (MODE == kGemmT) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 8 * (lane >> 5) + ((lane & 15) >> 2) + 4 * h;
        const int n = wt * WT + nb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        boff[nb][h] = kBV * kStageRowBytes + k * kBRowBytes + (((n >> 3) ^ bswizzle(k)) << 4) + (n & 7) * 2;
      }
  }
  auto read_b = [&](const char* sb, int kb) {
    if constexpr (MODE == kGemmT) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      FLCE_LDS const char* lb = (FLCE_LDS const char*)smem + (sb - smem);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (FLCE_LDS s16x4*)(lb + boff[nb][0] + kb * 16 * kBRowBytes));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (FLCE_LDS s16x4*)(lb + boff[nb][1] + kb * 16 * kBRowBytes));
        const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        fb[kb % kBSets][nb] = __builtin_bit_cast(Frag, v);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        fb[kb % kBSets][nb] = *(const Frag*)(sb + (b_row + nb * M) * kStageRowBytes + koff[kb]);
    }
  };
  constexpr int STEPS = NB * (sizeof(T) == 2 ? 1 : 4);  // matrix instructions per W fragment

  // ---- main loop over the chunk's stages (tile-major, k-stage minor); stage g
  // lives in LDS buffer g & 1 and takes QN MFMA steps (one W fragment each).
  //   steps [0, QN - kASlots): MFMAs, the fragment reads kASlots steps ahead,
  //     and this wave's remaining loads of stage g + 1 (into the other
  //     buffer), one per step;
  //   then the barrier: every wave's loads of stage g + 1 have landed, and
  //     every read of stage g has been issued and waited for;
  //   steps [QN - kASlots, QN): the last MFMAs of stage g, the first fragment
  //     reads of stage g + 1, and the first kASlots loads of stage g + 2 into
  //     stage g's buffer, which the barrier has just retired.
  // So the fragments the next stage starts with are read under this stage's
  // last MFMAs, not after the barrier with nothing to overlap, and the loads
  // go out one per step: issued all at once, the 8 waves' loads stall
  // instruction issue for a long stretch (the address path saturates); one per
  // step, a wave waiting to issue leaves the SIMD to the other wave's MFMAs.
  // Loads past the chunk's last stage read out of range (zero fill, no
  // memory traffic).
  static_assert(NLOADS > kASlots && NLOADS - kASlots <= QN - kASlots, "loads split over the steps");
  static_assert(!kTB || (NLOADS + 1) / 2 <= QN - kASlots, "transposed B: two loads a step");
  // prologue: all of stage 0, the first kASlots loads of stage 1
#pragma unroll
  for (int i = 0; i < NLOADS; ++i) issue_one(0, i, true);
  issue_done();
  if constexpr (!kTB) {
#pragma unroll
    for (int i = 0; i < kASlots; ++i) issue_one(1, i, 1 < total);
  }
  int* ysm = (int*)(smem + C::LDS_BYTES);  // kYLds: target of token t0 + t (minus v_off), -1 past N
  if constexpr (kYLds) {
    for (int t = threadIdx.x; t < kBT; t += C::THREADS) ysm[t] = t0 + t < p.N ? p.y[t0 + t] - p.v_off : -1;
  }
  FLCE_WAIT_VMCNT(0);
  __syncthreads();
  read_b(smem, 0);
#pragma unroll
  for (int q = 0; q < kASlots; ++q) read_a(smem, q);
  // Issue priority: the older wave of each SIMD (waves 0..NW/2-1) wins
  // arbitration by age, runs ahead and waits at the barrier while the younger
  // one feeds the matrix core alone. With YOUNG_PRIO the younger wave takes
  // the higher priority from the barrier through the stage's last steps (and
  // a tile's epilogue) and drops it when the next stage's main steps begin.
  const bool young = C::YOUNG_PRIO && wave >= C::NW / 2;
  int tile = 0;
  // One stage g of the chunk (stage g lives in LDS buffer g & 1 and takes QN
  // MFMA steps). A tile's first stage is a separate copy (first_stage true),
  // so that its first k-block can start from a zero accumulator.
  auto stage = [&](auto first_stage, const int g) {
      const char* sb = smem + (g & 1) * kStageBytes;
      const char* sn = smem + ((g + 1) & 1) * kStageBytes;  // at g == total - 1: read and ignored
      const bool more1 = g + 1 < total;
      if (young) __builtin_amdgcn_s_setprio(0);
      // The main steps [q0, q1): each W fragment's matrix instructions, then the
      // reads its slot (and, at a k-block's start, the idle H set) can take,
      // then a load, kept in that order by the scheduling barriers. With kFirst
      // (the first stage of a tile) the first k-block's matrix instructions take
      // a zero accumulator (an inline constant), which starts the tile without
      // clearing its accumulators.
      auto main_steps = [&](auto first_stage, auto q0_c, auto q1_c) {
        constexpr bool kFirst = decltype(first_stage)::value;
        constexpr int q0 = decltype(q0_c)::value, q1 = decltype(q1_c)::value;
#pragma unroll
        for (int q = q0; q < q1; ++q) {
          const int kb = q / MB, mb = q % MB;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = MmaT::step(fa[q % kASlots], fb[kb % kBSets][nb], (kFirst && kb == 0) ? kZeroAcc : acc[mb][nb]);
          if constexpr (kTB) {
            if (q == 0) {
              read_b(sb, 1);
              read_b(sb, 2);
              read_b(sb, 3);
            }
          } else {
            if (mb == 0 && kb + 1 < KSTEPS) read_b(sb, kb + 1);  // the other set was last used by k-block kb - 1
          }
          read_a(sb, q + kASlots);
          if constexpr (kTB) {
            if (2 * q < NLOADS) issue_one((g + 1) & 1, 2 * q, more1);
            if (2 * q + 1 < NLOADS) issue_one((g + 1) & 1, 2 * q + 1, more1);
          } else {
            if (q + kASlots < NLOADS) issue_one((g + 1) & 1, q + kASlots, more1);
          }
        }
#pragma unroll
        for (int q = q0; q < q1; ++q) {
          const int kb = q / MB, mb = q % MB;
          if (kTB && q == 0) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 6 * NB, 0);      // k-blocks 1-3 of B (two reads each)
            __builtin_amdgcn_sched_group_barrier(0x008, STEPS - 1, 0);
          } else if (!kTB && mb == 0 && kb + 1 < KSTEPS) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);          // next k-block's H fragments
            __builtin_amdgcn_sched_group_barrier(0x008, STEPS - 1, 0);
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, STEPS, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);             // one W fragment
          if (kTB && 2 * q + 1 < NLOADS)
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);           // two loads
          else if (kTB ? 2 * q < NLOADS : q + kASlots < NLOADS)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);           // one load
        }
      };
      typedef std::integral_constant<int, 0> Q0;
      typedef std::integral_constant<int, MB> QMB;
      typedef std::integral_constant<int, QN - kASlots> QEnd;
      main_steps(first_stage, Q0{}, QMB{});
      main_steps(std::false_type{}, QMB{}, QEnd{});
      // (after the ordering above: placed before it, this code lands in the
      // middle of the ordered region and the LDS reads lose their interleaving)
      issue_done();
      if (more1) {
        FLCE_WAIT_VMCNT(0);      // this wave's loads of stage g + 1 have landed in LDS
        __syncthreads();         // ... and everyone's; every read of stage g is done
      }
      if (young) __builtin_amdgcn_s_setprio(1);
      // the last kASlots steps. In the chunk's last stage there is no barrier
      // and the loads (zero fill) go to the other buffer, which no wave reads
      // any more; the fragments read from it there are never used.
      const bool more2 = g + 2 < total;
      const int tbuf = more1 ? (g & 1) : ((g + 1) & 1);
#pragma unroll
      for (int j = 0; j < kASlots; ++j) {
        const int q = QN - kASlots + j;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[q % MB][nb] = MmaT::step(fa[j], fb[(KSTEPS - 1) % kBSets][nb], acc[q % MB][nb]);
        if (j == 0) read_b(sn, 0);
        read_a(sn, j);
        if constexpr (!kTB) issue_one(tbuf, j, more2);
      }
#pragma unroll
      for (int j = 0; j < kASlots; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, STEPS, 0);
        if (j == 0) __builtin_amdgcn_sched_group_barrier(0x100, (kTB ? 2 * NB : NB) + 1, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if constexpr (!kTB) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
  };
  for (int g = 0; g < total;) {
    stage(std::true_type{}, g++);
    for (int ks = 1; ks < KS; ++ks) stage(std::false_type{}, g++);

    const int vw = (tile_begin + tile) * kBV + a_row;   // first A row (vocabulary row) of this wave
    ++tile;
    if constexpr (MODE == kForward) {
      // ---- epilogue of one vocabulary tile, entirely in registers. The
      // lane's index is taken afresh here (mbcnt on an opaque all-ones mask,
      // so that nothing derived from it is hoisted and kept live across the
      // stage loop, where it had been spilled).
      unsigned all = ~0u;
      asm volatile("" : "+s"(all));
      const int ln = (int)__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u));
      if (vw + WV > p.V) {
        // ragged last tile: vocabulary rows >= V are not logits at all
        int lim = p.V - vw - 4 * (ln / M);
        asm volatile("" : "+v"(lim));  // compared here, not hoisted as per-register lane masks
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < ACC; ++r)
              if (mb * M + row_in(r) >= lim) acc[mb][nb][r] = kNegInf;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // target logit: written by the one lane holding (y, token), in this (rare, divergent) branch
        const int rel = (kYLds ? ysm[wt * WT + nb * M + (ln % M)] : ytok[nb]) - vw;
        if ((unsigned)rel < (unsigned)WV && ((rel >> 2) & (64 / M - 1)) == ln / M) {
          int want = rel;
          asm volatile("" : "+v"(want));  // likewise
          const int want_mb = want / M;
          const int want_r = M == 32 ? ((want & 31) >> 3) * 4 + (want & 3) : (want & 3);
          float val = 0.f;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < ACC; ++r)
              if (mb == want_mb && r == want_r) val = acc[mb][nb][r];
          p.z_target[t0 + wt * WT + nb * M + (ln % M)] = val;
        }
        // online update: m' = max(m, m_tile), s' = s e^(m - m') + sum_j e^(z_j - m')
        float tmax = kNegInf;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < ACC; ++r) tmax = fmaxf(tmax, acc[mb][nb][r]);
        const float m_old = kMLds ? msm[nb * 64] : m_run[nb];
        const float m_new = fmaxf(m_old, tmax);
        const float c = (m_new == kNegInf) ? 0.f : off2(m_new);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < ACC; r += 2) {
            s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][r], kLog2e, -c));
            s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][r + 1], kLog2e, -c));
          }
        s_run[nb] = s_run[nb] * __builtin_amdgcn_exp2f(off2(m_old) - c) + (s0 + s1);
        if constexpr (kMLds)
          msm[nb * 64] = m_new;
        else
          m_run[nb] = m_new;
      }
    } else if constexpr (MODE == kDz) {
      // ---- dZ = g (softmax(Z) - onehot(y)) of one tile, with
      // softmax = 2^(z log2(e) - lse log2(e)); rows >= V and tokens >= N are 0.
      // Written to dz[tok][v] (four consecutive v per lane and register group)
      // and dzt[v][tok] (M consecutive tokens per M lanes).
      const int v_lane = vw + lane_row;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int tok = t0 + wt * WT + nb * M + (lane % M);
        if (tok >= p.dz_rows) continue;
        const bool tok_ok = tok < p.N;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r4 = 0; r4 < ACC / 4; ++r4) {
            const int v0 = v_lane + mb * M + 8 * r4;   // rows v0 .. v0 + 3 in registers 4*r4 ..
            if (v0 >= p.dz_cols) continue;
            T q[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int v = v0 + j;
              float d = 0.f;
              if (tok_ok && v < p.V) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][4 * r4 + j], kLog2e, -l2tok[nb]));
                d = gtok[nb] * (v == ytok[nb] ? e - 1.f : e);
              }
              q[j] = (T)d;
              *(T*)(p.dzt + ((size_t)v * p.dzt_ld + tok) * sizeof(T)) = q[j];
            }
            if (p.dz) store4(p.dz + ((size_t)tok * p.dz_ld + v0) * sizeof(T), q);
          }
      }
    } else if constexpr (MODE == kGemmT) {
      // ---- C[b][a] = Z (or C[b][a] + Z) for a < V, b < N: four consecutive a
      // per lane and register group, one 16-byte store each
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int b = t0 + wt * WT + nb * 32 + (lane & 31);
        if (b >= p.N) continue;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int a0 = vw + mb * 32 + 8 * r4 + lane_row;
            if (a0 >= p.V) continue;
            float q[4] = {acc[mb][nb][4 * r4], acc[mb][nb][4 * r4 + 1], acc[mb][nb][4 * r4 + 2],
                          acc[mb][nb][4 * r4 + 3]};
            float* dst = p.C + ((size_t)kslice * p.N + b) * p.ldc + a0;
            if (p.accumulate) {
              const f32x4 old = *(const f32x4*)dst;
#pragma unroll
              for (int j = 0; j < 4; ++j) q[j] = old[j] + q[j];
            }
            store4((char*)dst, q);
          }
      }
    } else {
      // ---- C[a][b] = Z (or C[a][b] + Z) for a < V, b < N
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int b = t0 + wt * WT + nb * M + (lane % M);
        if (b >= p.N) continue;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < ACC; ++r) {
            const int a = vw + mb * M + row_in(r) + lane_row;
            if (a < p.V) {
              float* dst = p.C + (size_t)a * p.ldc + b;
              *dst = p.accumulate ? *dst + acc[mb][nb][r] : acc[mb][nb][r];
            }
          }
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
  FLCE_WAIT_VMCNT(0);  // the last stage's zero-filling loads land before the workgroup ends


  if constexpr (MODE != kForward) return;

  if constexpr (kMLds) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) m_run[nb] = msm[nb * 64];
  }
  // ---- end of chunk: combine the 64 / M lanes that hold the same token
  // column (xor M, then xor 2M), then the kWavesV waves that share a token
  // range, in a fixed order (deterministic), and write one (m, s) per token.
#pragma unroll
  for (int x = M; x < 64; x *= 2)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float m2 = __shfl_xor(m_run[nb], x);
      const float s2 = __shfl_xor(s_run[nb], x);
      combine(m_run[nb], s_run[nb], m2, s2);
    }
  __syncthreads();  // every wave is done with the stage buffers
  float* red = (float*)smem;  // [kWavesV][kBT] m, then [kWavesV][kBT] s
  if (lane < M) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wt * WT + nb * M + lane;
      red[wv * kBT + col] = m_run[nb];
      red[(kWavesV + wv) * kBT + col] = s_run[nb];
    }
  }
  __syncthreads();
  if (wv == 0 && lane < M) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wt * WT + nb * M + lane;
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

template <typename T, typename C>
__global__ __launch_bounds__(C::THREADS, 1) void flce_partials_kernel(TileArgs p) {
  tile_loop<T, C, kForward>(p);
}

template <typename T, typename C>
__global__ __launch_bounds__(C::THREADS, 1) void flce_dz_kernel(TileArgs p) {
  tile_loop<T, C, kDz>(p);
}

template <typename T, typename C>
__global__ __launch_bounds__(C::THREADS, 1) void flce_gemm_kernel(TileArgs p) {
  tile_loop<T, C, kGemm>(p);
}

template <typename T, typename C>
__global__ __launch_bounds__(C::THREADS, 1) void flce_gemmt_kernel(TileArgs p) {
  tile_loop<T, C, kGemmT>(p);
}

// Merge: one thread per token. With off(m) = fl(m log2 e) as in the partials
// kernel, C = max_c off(m_c), S = sum_c s_c 2^(off(m_c) - C),
// lse = (C + log2 S) ln 2 and loss = lse - z_y (NaN when y is not in [0, V)).
// C is a maximum of fp32 values (exact); each weight 2^(off(m_c) - C) is the
// hardware fp32 exp2 of the difference (relative error ~1e-6 for every weight
// above 2^-30, far below the partial sums' own rounding); S and the final
// logarithm are carried in double. A NaN in m or s reaches S and the row's
// lse and loss.
constexpr int kMergeThreads = 64;
__global__ __launch_bounds__(kMergeThreads) void flce_merge_kernel(const float* __restrict__ part_m,
                                                                   const float* __restrict__ part_s,
                                                                   const float* __restrict__ z_target,
                                                                   const int32_t* __restrict__ y, int N, int V,
                                                                   int chunks, float* __restrict__ loss,
                                                                   float* __restrict__ lse) {
  const int i = blockIdx.x * kMergeThreads + threadIdx.x;
  if (i >= N) return;
  float C = kNegInf;
  for (int c = 0; c < chunks; ++c) C = fmaxf(C, off2(part_m[(size_t)c * N + i]));
  double S = 0.0;
#pragma unroll 4
  for (int c = 0; c < chunks; ++c) {
    const float o = off2(part_m[(size_t)c * N + i]);
    const float w = (o == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(o - C);
    S += (double)part_s[(size_t)c * N + i] * (double)w;
  }
  const double l = ((double)C + log2(S)) * 0.69314718055994530942;
  if (lse) lse[i] = (float)l;
  const int t = y[i];
  loss[i] = (t >= 0 && t < V) ? (float)(l - (double)z_target[i]) : __builtin_nanf("");
}

// ------------------------------------------------------------------ backward helpers
// out[c][r] = in[r][c] for c < cols and r < rows, and 0 for rows <= r < out_len:
// the backward's K-contiguous copies of W (vocabulary along K) and of H (tokens
// along K). 64 x 64 tiles staged through LDS, moved in 16-byte vectors both
// ways (cols, ld_in, out_len and ld_out are multiples of 16 bytes' worth of
// elements). The LDS row is padded by 4 bytes, so the column gathers of one
// store instruction (8 rows 8 apart x 8 columns) fall on distinct banks.
template <typename T>
__global__ __launch_bounds__(256) void flce_transpose_kernel(const T* __restrict__ in, int rows, int cols,
                                                             int64_t ld_in, T* __restrict__ out,
                                                             int64_t ld_out, int out_len) {
  constexpr int E = 16 / sizeof(T);      // elements per 16-byte vector
  constexpr int VPR = 64 / E;            // vectors per 64-element tile row
  constexpr int PAD = 4 / sizeof(T) > 0 ? 4 / sizeof(T) : 1;
  typedef T vec __attribute__((ext_vector_type(E)));
  __shared__ T tile[64][64 + PAD];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  // load: tile row i, elements [E*j, E*j + E)
#pragma unroll
  for (int k = threadIdx.x; k < 64 * VPR; k += 256) {
    const int i = k / VPR, j = k % VPR;
    const int r = r0 + i, c = c0 + E * j;
    vec v = {};
    if (r < rows && c < cols) v = *(const vec*)(in + (size_t)r * ld_in + c);
#pragma unroll
    for (int e = 0; e < E; ++e) tile[i][E * j + e] = v[e];
  }
  __syncthreads();
  // store: out row c0 + i (tile column i), elements [r0 + E*j, + E)
#pragma unroll
  for (int k = threadIdx.x; k < 64 * VPR; k += 256) {
    const int i = k / VPR, j = k % VPR;
    const int c = c0 + i, r = r0 + E * j;
    if (c >= cols || r >= out_len) continue;
    vec v;
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = tile[E * j + e][i];
    *(vec*)(out + (size_t)c * ld_out + r) = v;
  }
}

// dst[0..n) = 0.
__global__ __launch_bounds__(256) void flce_zero_kernel(float* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = 0.f;
}

// Sum of the S partial products of a split dH product, in order (so the
// result does not depend on scheduling), written to out or, with accumulate,
// added to it. n4 = elements / 4.
__global__ __launch_bounds__(256) void flce_ksum_kernel(const float* __restrict__ part, int S, int64_t n4,
                                                        float* __restrict__ out, int accumulate) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 acc = ((const f32x4*)part)[i];
    if (accumulate) acc = ((const f32x4*)out)[i] + acc;
    for (int s = 1; s < S; ++s) acc += ((const f32x4*)part)[(int64_t)s * n4 + i];
    ((f32x4*)out)[i] = acc;
  }
}

// Quantised output head: rows [0, rows) of the codes, dequantised to bf16.
// Each thread turns 8 consecutive weights of a row (8 code bytes at 8 bits; 4
// bytes at 4 bits, byte k holding weight 2k in its low nibble and 2k + 1 in
// its high one) into 16 bytes of bf16, w = bf16(fl(fl(scale * q) + bias)) with
// the scale and bias of the weights' group (group % 8 == 0, so the 8 share
// one). Consecutive lanes write consecutive 16 bytes, so the stores, which
// are most of the traffic, coalesce; giving a thread 16 or 32 weights (wider
// code loads) broke that and was slower.
template <int BITS>
__global__ __launch_bounds__(256) void flce_dequant_kernel(const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales,
                                                           const float* __restrict__ biases, int64_t rows,
                                                           int D, int group, __bf16* __restrict__ out) {
  const int per_row = D / 8;
  const int groups = D / group;
  const int64_t n = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row;
    const int d0 = (int)(i - r * per_row) * 8;
    const int64_t gi = r * groups + d0 / group;
    const float sc = scales[gi], bi = biases[gi];
    uint32_t q[8];
    if constexpr (BITS == 8) {
      const uint2 v = *(const uint2*)(codes + r * D + d0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        q[k] = (v.x >> (8 * k)) & 0xFFu;
        q[k + 4] = (v.y >> (8 * k)) & 0xFFu;
      }
    } else {
      const uint32_t v = *(const uint32_t*)(codes + r * (D / 2) + d0 / 2);
#pragma unroll
      for (int k = 0; k < 8; ++k) q[k] = (v >> (4 * k)) & 0xFu;
    }
    bf16x8 w;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float prod = (float)q[k] * sc;
      w[k] = (__bf16)(prod + bi);
    }
    *(bf16x8*)(out + r * D + d0) = w;
  }
}

// ------------------------------------------------------------------ host side
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

// Arguments of the tile loop for a plan: B rows (H role) x A rows (W role),
// both row_bytes long.
TileArgs tile_args(const Plan& pl, const void* B, const void* A) {
  TileArgs a;
  memset(&a, 0, sizeof a);
  a.H = (const char*)B;
  a.W = (const char*)A;
  a.N = pl.N;
  a.V = pl.V;
  a.row_bytes = pl.row_bytes;
  a.row_blocks = pl.row_blocks;
  a.vocab_tiles = pl.vocab_tiles;
  a.chunks = pl.chunks;
  a.xcd_rows = pl.xcd_rows;
  a.xcd_chunks = pl.xcd_chunks;
  return a;
}

// Launch KERNEL<T, Tile> for the plan's dtype and tile (fp32 runs 256x256 only).
#define FLCE_LAUNCH_TILES(KERNEL, pl, args, stream)                                                     \
  do {                                                                                                  \
    if ((pl).dtype == FLCE_FP32)                                                                        \
      hipLaunchKernelGGL((KERNEL<float, Tile256>), dim3((pl).grid), dim3(Tile256::THREADS), 0, stream, args);  \
    else if ((pl).tile == kTile384)                                                                     \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile384>), dim3((pl).grid), dim3(Tile384::THREADS), 0, stream, args); \
    else if ((pl).tile == kTile320)                                                                     \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile320h>), dim3((pl).grid), dim3(Tile320h::THREADS), 0, stream, args); \
    else                                                                                                \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile256h>), dim3((pl).grid), dim3(Tile256h::THREADS), 0, stream, args); \
  } while (0)

// The backward's launches: 32x32 tiles for every tile id.
#define FLCE_LAUNCH_TILES_M32(KERNEL, pl, args, stream)                                                 \
  do {                                                                                                  \
    if ((pl).dtype == FLCE_FP32)                                                                        \
      hipLaunchKernelGGL((KERNEL<float, Tile256>), dim3((pl).grid), dim3(Tile256::THREADS), 0, stream, args);  \
    else if ((pl).tile == kTile384)                                                                     \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile384>), dim3((pl).grid), dim3(Tile384::THREADS), 0, stream, args); \
    else if ((pl).tile == kTile320)                                                                     \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile320>), dim3((pl).grid), dim3(Tile320::THREADS), 0, stream, args); \
    else                                                                                                \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile256>), dim3((pl).grid), dim3(Tile256::THREADS), 0, stream, args); \
  } while (0)

// The transposed-B product: bf16 only, and at most the 320-row tile (its four
// sets of B fragments do not fit the 384-row tile's registers).
#define FLCE_LAUNCH_TILES_GEMMT(KERNEL, pl, args, stream)                                               \
  do {                                                                                                  \
    if ((pl).tile == kTile320)                                                                          \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile320>), dim3((pl).grid), dim3(Tile320::THREADS), 0, stream, args); \
    else                                                                                                \
      hipLaunchKernelGGL((KERNEL<__bf16, Tile256>), dim3((pl).grid), dim3(Tile256::THREADS), 0, stream, args); \
  } while (0)

int launch_partials(const Plan& pl, const void* H, const void* W, const int32_t* y, void* ws,
                    hipStream_t stream) {
  TileArgs a = tile_args(pl, H, W);
  a.y = y;
  a.part_m = (float*)((char*)ws + pl.off_m);
  a.part_s = (float*)((char*)ws + pl.off_s);
  a.z_target = (float*)((char*)ws + pl.off_z);
  FLCE_LAUNCH_TILES(flce_partials_kernel, pl, a, stream);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int launch_merge(const Plan& pl, const int32_t* y, float* loss, float* lse, const void* ws,
                 hipStream_t stream) {
  const float* m = (const float*)((const char*)ws + pl.off_m);
  const float* s = (const float*)((const char*)ws + pl.off_s);
  const float* z = (const float*)((const char*)ws + pl.off_z);
  hipLaunchKernelGGL(flce_merge_kernel, dim3((pl.N + kMergeThreads - 1) / kMergeThreads), dim3(kMergeThreads), 0,
                     stream, m, s, z, y,
                     pl.N, pl.V, pl.chunks, loss, lse);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// ------------------------------------------------------------------ backward
// The backward runs the vocabulary in slices of Vs rows, so that dZ only ever
// exists for one slice. Per slice s (rows [v0, v0 + Vs) of W, Vsp = Vs
// rounded up to 64):
//   1. W_s^T ([D][Vsp]), the K-contiguous A operand of dH (transpose kernel);
//   2. the dZ pass recomputes Z for all rows over the slice's vocabulary (the
//      forward's tile loop on W rows [v0, v0 + Vs), targets offset by v0) and
//      writes dZ_s = g (softmax - onehot), rounded to the input dtype,
//      transposed: dzt[Vsp][Np] (for fp32 also row-major: dz[Np][Vsp]);
//   3. dH (+)= dZ_s W_s: bf16 reads dZ_s from dzt through transposing LDS
//      reads (A = W_s^T, B = dzt); fp32 has no transposing 32-bit read and
//      uses the row-major copy (A = dz, B = W_s^T). The first slice writes dH,
//      later slices add to it, in slice order (deterministic). When the bf16
//      product's tiles would leave compute units idle, its contraction is
//      split again into float32 partial sums that flce_ksum_kernel adds in
//      order;
//   4. dW[v0, v0 + Vs) = dzt . H (A = dzt, B = H^T [D][Np], transposed once
//      per call): each slice owns its rows of dW, nothing is accumulated.
// Vs is the largest size (balanced over the slices) whose dZ buffers fit
// kDzBudget bytes, one transposed copy for bf16 and two copies for fp32, so
// the workspace is W_s^T + H^T + at most kDzBudget of dZ (+ the bf16 split's
// partial sums at shapes too small to fill the chip): it grows with V D and
// N D, never with N V. Padding rows and columns (to 64 elements, so that rows
// of the transposed copies start on 128-byte lines) are written as zeros, so
// the products need no masks on K.

template <typename T>
void launch_transpose(const void* in, int rows, int cols, int64_t ld_in, void* out, int64_t ld_out,
                      int out_len, hipStream_t stream) {
  const dim3 grid((unsigned)((out_len + 63) / 64), (unsigned)((cols + 63) / 64));
  hipLaunchKernelGGL((flce_transpose_kernel<T>), grid, dim3(256), 0, stream, (const T*)in, rows, cols, ld_in,
                     (T*)out, ld_out, out_len);
}

void launch_ksum(const float* part, int S, int64_t n, float* out, bool accumulate, hipStream_t stream) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(flce_ksum_kernel, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 2048)), dim3(256), 0,
                     stream, part, S, n4, out, accumulate ? 1 : 0);
}

// Buffers of a backward call, in the workspace.
struct BwdBuffers {
  char* wt;     // W_s^T [D][Vsp]
  char* ht;     // H^T [D][Np] (only when dW is wanted)
  char* dzt;    // dZ_s^T [Vsp][Np]
  char* dz;     // dZ_s [Np][Vsp] (fp32 only)
  float* part;  // bf16 split dH partial sums
};

// Steps 1-4 for one slice: Ws = W rows [v0, v0 + Vs); dH is written
// (first) or added to; dWs (rows [v0, v0 + Vs) of dW) is written when not null.
void backward_slice(const SlicePlans& sp, int dtype, int64_t N, int64_t D, int64_t Np, const void* H,
                    const void* Ws, int64_t v0, const int32_t* y, const float* lse, const float* grad, float* dH,
                    bool first, float* dWs, const BwdBuffers& b, hipStream_t stream) {
  const bool bf = dtype == FLCE_BF16;
  if (bf)
    launch_transpose<__bf16>(Ws, (int)sp.Vs, (int)D, D, b.wt, sp.Vsp, (int)sp.Vsp, stream);
  else
    launch_transpose<float>(Ws, (int)sp.Vs, (int)D, D, b.wt, sp.Vsp, (int)sp.Vsp, stream);
  // dZ of the slice: dzt columns [0, Np) and rows [0, Vsp) (padding as zeros)
  TileArgs a = tile_args(sp.dz, H, Ws);
  a.y = y;
  a.v_off = (int)v0;
  a.lse = lse;
  a.grad = grad;
  a.dz = bf ? nullptr : b.dz;
  a.dzt = b.dzt;
  a.dz_ld = (int)sp.Vsp;
  a.dzt_ld = (int)Np;
  a.dz_rows = (int)Np;
  a.dz_cols = (int)sp.Vsp;
  FLCE_LAUNCH_TILES_M32(flce_dz_kernel, sp.dz, a, stream);
  if (bf) {
    // dH[token][d] (+)= sum_v dZ[token][v] W_s[v][d]: A = W_s^T, B = dZ read from dzt
    TileArgs g = tile_args(sp.dh, b.dzt, b.wt);
    g.ldb = (int)Np;
    g.ldc = (int)D;
    g.ksplit = sp.ksplit;
    g.ks_per = sp.ks_per;
    g.C = sp.ksplit > 1 ? b.part : dH;
    g.accumulate = (sp.ksplit == 1 && !first) ? 1 : 0;
    Plan phs = sp.dh;
    phs.grid = sp.dh.row_blocks * sp.dh.chunks * sp.ksplit;
    FLCE_LAUNCH_TILES_GEMMT(flce_gemmt_kernel, phs, g, stream);
    if (sp.ksplit > 1) launch_ksum(b.part, sp.ksplit, N * D, dH, !first, stream);
  } else {
    // dH[token][d] (+)= sum_v dz[token][v] W_s^T[d][v]: A = dz, B = W_s^T
    TileArgs g = tile_args(sp.dh, b.wt, b.dz);
    g.C = dH;
    g.ldc = (int)D;
    g.accumulate = first ? 0 : 1;
    FLCE_LAUNCH_TILES_M32(flce_gemm_kernel, sp.dh, g, stream);
  }
  if (dWs) {
    // dW_s[v][d] = sum_token dzt[v][token] H^T[d][token]: A = dzt, B = H^T
    TileArgs w = tile_args(sp.dw, b.ht, b.dzt);
    w.C = dWs;
    w.ldc = (int)D;
    FLCE_LAUNCH_TILES_M32(flce_gemm_kernel, sp.dw, w, stream);
  }
}

int launch_backward(const BwdPlan& bp, const void* H, const void* W, const int32_t* y, const float* lse,
                    const float* grad, float* dH, float* dW, void* ws, hipStream_t stream) {
  if (bp.slices == 0) {  // no rows: dW = 0
    const int64_t n = bp.V * bp.D;
    hipLaunchKernelGGL(flce_zero_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0,
                       stream, dW, n);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  char* base = (char*)ws;
  const BwdBuffers b = {base + bp.off_wt, base + bp.off_ht, base + bp.off_dzt, base + bp.off_dz,
                        (float*)(base + bp.off_part)};
  if (bp.dtype == FLCE_BF16)
    launch_transpose<__bf16>(H, (int)bp.N, (int)bp.D, bp.D, b.ht, bp.Np, (int)bp.Np, stream);
  else
    launch_transpose<float>(H, (int)bp.N, (int)bp.D, bp.D, b.ht, bp.Np, (int)bp.Np, stream);
  for (int s = 0; s < bp.slices; ++s) {
    const SlicePlans& sp = s + 1 < bp.slices ? bp.full : bp.last;
    const int64_t v0 = (int64_t)s * bp.Vs;
    backward_slice(sp, bp.dtype, bp.N, bp.D, bp.Np, H, (const char*)W + v0 * bp.D * (int64_t)bp.es, v0, y, lse,
                   grad, dH, s == 0, dW + v0 * bp.D, b, stream);
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// ------------------------------------------------------------------ quantised head
// The vocabulary runs in slices of Vs rows: each slice is dequantised into a
// bf16 buffer in the workspace and run through the partials kernel with its
// chunks' partial states written after the previous slices' (and targets
// offset by the slice's first row), then one merge covers every chunk. Vs is
// a multiple of 3072 rows (8 chunks of whole 384-row tiles; 30720 rows at
// D = 4096 also split evenly into 320- and 256-row tiles) with the buffer
// near kQuantSliceBytes; a vocabulary that fits one slice is a single pass.
void launch_dequant(int bits, int D, int group, const uint8_t* codes, const float* scales, const float* biases,
                    int64_t rows, __bf16* out, hipStream_t stream) {
  const int64_t n = rows * (D / 8);
  const dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, 8192)), block(256);
  if (bits == 8)
    hipLaunchKernelGGL((flce_dequant_kernel<8>), grid, block, 0, stream, codes, scales, biases, rows, D, group, out);
  else
    hipLaunchKernelGGL((flce_dequant_kernel<4>), grid, block, 0, stream, codes, scales, biases, rows, D, group, out);
}

int launch_forward_quant(const QuantPlan& qp, const void* H, const uint8_t* codes, const float* scales,
                         const float* biases, const int32_t* y, float* loss, float* lse, void* ws,
                         hipStream_t stream) {
  char* base = (char*)ws;
  __bf16* buf = (__bf16*)(base + qp.off_buf);
  float* m = (float*)(base + qp.off_m);
  float* s = (float*)(base + qp.off_s);
  float* z = (float*)(base + qp.off_z);
  const size_t code_row = (size_t)(qp.bits == 8 ? qp.D : qp.D / 2);
  const int64_t groups = qp.D / qp.group;
  int64_t c0 = 0;
  for (int k = 0; k < qp.slices; ++k) {
    const Plan& pl = k + 1 < qp.slices ? qp.full : qp.last;
    const int64_t v0 = (int64_t)k * qp.Vs;
    const int64_t rows = pl.V;
    launch_dequant(qp.bits, (int)qp.D, qp.group, codes + v0 * code_row, scales + v0 * groups, biases + v0 * groups,
                   rows, buf, stream);
    TileArgs a = tile_args(pl, H, buf);
    a.y = y;
    a.v_off = (int)v0;
    a.part_m = m + c0 * qp.N;
    a.part_s = s + c0 * qp.N;
    a.z_target = z;
    FLCE_LAUNCH_TILES(flce_partials_kernel, pl, a, stream);
    c0 += pl.chunks;
  }
  hipLaunchKernelGGL(flce_merge_kernel, dim3((unsigned)((qp.N + kMergeThreads - 1) / kMergeThreads)),
                     dim3(kMergeThreads), 0, stream, (const float*)m, (const float*)s, (const float*)z, y,
                     (int)qp.N, (int)qp.V, qp.chunks_total, loss, lse);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// Backward of the quantised-head forward for a frozen head: dH only. The
// vocabulary runs in slices as in the dense backward (backward_slice without
// dW), each first dequantised into the workspace; a slice is at most the
// forward's dequantisation slice and keeps dZ^T within kDzBudget.
int launch_backward_quant(const QuantBwdPlan& qb, const void* H, const uint8_t* codes, const float* scales,
                          const float* biases, const int32_t* y, const float* lse, const float* grad, float* dH,
                          void* ws, hipStream_t stream) {
  char* base = (char*)ws;
  __bf16* wbuf = (__bf16*)(base + qb.off_w);
  const BwdBuffers b = {base + qb.off_wt, nullptr, base + qb.off_dzt, nullptr, (float*)(base + qb.off_part)};
  const size_t code_row = (size_t)(qb.bits == 8 ? qb.D : qb.D / 2);
  const int64_t groups = qb.D / qb.group;
  for (int k = 0; k < qb.slices; ++k) {
    const SlicePlans& sp = k + 1 < qb.slices ? qb.full : qb.last;
    const int64_t v0 = (int64_t)k * qb.Vs;
    launch_dequant(qb.bits, (int)qb.D, qb.group, codes + v0 * code_row, scales + v0 * groups, biases + v0 * groups,
                   sp.Vs, wbuf, stream);
    backward_slice(sp, FLCE_BF16, qb.N, qb.D, qb.Np, H, wbuf, v0, y, lse, grad, dH, k == 0, nullptr, b, stream);
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// ------------------------------------------------------------------ static scratch
// flce_forward_noalloc's workspace: a file-scope device array, one copy per
// GPU, held until the process ends. Host code never uses the array's name as
// an address (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and is what the kernels receive.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the device's first use).
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return FLCE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FLCE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return FLCE_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
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
    case FLCE_ERR_SCRATCH: return "shape needs more workspace than the static scratch holds (16 MiB)";
    default: return "unknown status";
  }
}

int flce_get_plan(int64_t N, int64_t D, int64_t V, int dtype, flce_plan_t* out) {
  if (!out) return FLCE_ERR_INVALID_ARG;
  Plan pl;
  const int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return rc;
  out->tile_vocab = pl.BV;
  out->tile_tokens = pl.BT;
  out->row_blocks = pl.row_blocks;
  out->vocab_tiles = pl.vocab_tiles;
  out->chunks = pl.chunks;
  out->grid = N > 0 ? pl.grid : 0;
  out->xcd_rows = pl.xcd_rows;
  out->xcd_chunks = pl.xcd_chunks;
  out->threads = pl.threads;
  out->lds_bytes = pl.lds_bytes;
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

int flce_forward_noalloc(const void* H, const void* W, const int32_t* targets, int64_t N, int64_t D, int64_t V,
                         int dtype, float* loss_out, float* lse_out, void* stream) {
  Plan pl;
  int rc = make_plan(N, D, V, dtype, &pl);
  if (rc != FLCE_OK) return rc;
  if ((rc = check_inputs(H, W, targets, N)) != FLCE_OK) return rc;
  if (N == 0) return FLCE_OK;
  if (!loss_out || !aligned(loss_out, 4) || (lse_out && !aligned(lse_out, 4)))
    return FLCE_ERR_INVALID_ARG;
  if (pl.ws_bytes > kScratchBytes) return FLCE_ERR_SCRATCH;
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws)) != FLCE_OK) return rc;
  // Every partial the merge reads (m and s per row and chunk, and the target
  // logit of each row whose target is in [0, V)) is written by the partials
  // launch of the same call, so nothing in the scratch needs clearing.
  hipStream_t s = (hipStream_t)stream;
  if ((rc = launch_partials(pl, H, W, targets, ws, s)) != FLCE_OK) return rc;
  return launch_merge(pl, targets, loss_out, lse_out, ws, s);
}

size_t flce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype) {
  BwdPlan bp;
  if (make_bwd_plan(N, D, V, dtype, &bp) != FLCE_OK) return 0;
  return bp.ws_bytes;
}

int flce_backward(const void* H, const void* W, const int32_t* targets, const float* lse, const float* grad_loss,
                  int64_t N, int64_t D, int64_t V, int dtype, float* dH, float* dW, void* workspace,
                  size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  int rc = make_bwd_plan(N, D, V, dtype, &bp);
  if (rc != FLCE_OK) return rc;
  if (!W || !dW || !aligned(W, 16) || !aligned(dW, 4)) return FLCE_ERR_INVALID_ARG;
  if (N > 0) {
    if ((rc = check_inputs(H, W, targets, N)) != FLCE_OK) return rc;
    if (!lse || !grad_loss || !dH || !aligned(lse, 4) || !aligned(grad_loss, 4) || !aligned(dH, 16))
      return FLCE_ERR_INVALID_ARG;
  }
  if (!workspace || workspace_bytes < bp.ws_bytes || !aligned(workspace, kAlign)) return FLCE_ERR_INVALID_ARG;
  return launch_backward(bp, H, W, targets, lse, grad_loss, dH, dW, workspace, (hipStream_t)stream);
}

size_t flce_forward_quant_workspace_bytes(int64_t N, int64_t D, int64_t V, int bits, int group) {
  QuantPlan qp;
  if (N == 0 || make_quant_plan(N, D, V, bits, group, &qp) != FLCE_OK) return 0;
  return qp.ws_bytes;
}

int flce_forward_quant(const void* H, const uint8_t* codes, const float* scales, const float* biases,
                       const int32_t* targets, int64_t N, int64_t D, int64_t V, int bits, int group,
                       float* loss_out, float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  QuantPlan qp;
  int rc = make_quant_plan(N, D, V, bits, group, &qp);
  if (rc != FLCE_OK) return rc;
  if (N == 0) return FLCE_OK;
  if (!H || !codes || !scales || !biases || !targets || !loss_out) return FLCE_ERR_INVALID_ARG;
  if (!aligned(H, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(biases, 4) ||
      !aligned(targets, 4) || !aligned(loss_out, 4) || (lse_out && !aligned(lse_out, 4)))
    return FLCE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < qp.ws_bytes || !aligned(workspace, kAlign)) return FLCE_ERR_INVALID_ARG;
  return launch_forward_quant(qp, H, codes, scales, biases, targets, loss_out, lse_out, workspace,
                              (hipStream_t)stream);
}

size_t flce_backward_quant_workspace_bytes(int64_t N, int64_t D, int64_t V, int bits, int group) {
  QuantBwdPlan qb;
  if (N == 0 || make_quant_bwd_plan(N, D, V, bits, group, &qb) != FLCE_OK) return 0;
  return qb.ws_bytes;
}

int flce_backward_quant(const void* H, const uint8_t* codes, const float* scales, const float* biases,
                        const int32_t* targets, const float* lse, const float* grad_loss, int64_t N, int64_t D,
                        int64_t V, int bits, int group, float* dH, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (N == 0) {
    QuantPlan q;
    return make_quant_plan(N, D, V, bits, group, &q);
  }
  QuantBwdPlan qb;
  int rc = make_quant_bwd_plan(N, D, V, bits, group, &qb);
  if (rc != FLCE_OK) return rc;
  if (!H || !codes || !scales || !biases || !targets || !lse || !grad_loss || !dH) return FLCE_ERR_INVALID_ARG;
  if (!aligned(H, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(biases, 4) ||
      !aligned(targets, 4) || !aligned(lse, 4) || !aligned(grad_loss, 4) || !aligned(dH, 16))
    return FLCE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < qb.ws_bytes || !aligned(workspace, kAlign)) return FLCE_ERR_INVALID_ARG;
  return launch_backward_quant(qb, H, codes, scales, biases, targets, lse, grad_loss, dH, workspace,
                               (hipStream_t)stream);
}

}  // extern "C"
