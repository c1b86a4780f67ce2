// Matrix-core ceiling of an MI355X (gfx950) for bf16: how many
// v_mfma_f32_32x32x16_bf16 per second the chip sustains with operands held
// in registers (no memory traffic at all), and at what shader clock.
//
// This is a measuring instrument beside the library, not part of the
// cross-entropy path. The forward's contraction (the page "Een gefuseerde
// forward-kernel voor lineaire cross-entropy op Apple-GPU's", section 1: the
// logits are the product of the hidden states and the output projection) runs
// on the same instruction, so its rate here bounds what any kernel built on it
// can reach on the same part: the nominal peak assumes 2.4 GHz, and under a
// sustained matrix-core load the part holds a lower clock.
//
// Each wave keeps 8 accumulators (32x32 fp32) and 4 A and 4 B operand
// fragments, loaded once from the caller's buffer (random values toggle the
// datapath as real data does; a constant buffer does not), and issues
// 32 MFMAs per iteration: accumulator j takes A fragment (j + k) % 4 and B
// fragment (k + 2j) % 4 for k = 0..3, so consecutive instructions always
// differ in both operands. Two issue orders of the same 32 instructions:
//   order 0: k outer, j inner -- consecutive MFMAs write different
//            accumulators (as in the forward's tile loop);
//   order 1: j outer, k inner -- each accumulator takes its 4 MFMAs back to
//            back (a dependent chain on one accumulator);
//   orders 2 and 3: as order 0, with the A operand (2) or both operands (3)
//            held for the 8 instructions of a k step, to measure what
//            operand toggling between instructions costs;
//   order 4: the same FLOP on v_mfma_f32_16x16x32_bf16 (16x16 outputs, K =
//            32, half the FLOP of one 32x32x16), twice as many instructions.
// Lane 0 of each workgroup records s_memtime (shader clock) and
// s_memrealtime (the fixed 100 MHz reference) before and after its loop, so
// the host can state the clock the part held.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_ceiling.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int ORDER>
__global__ __launch_bounds__(512, 1) void flce_ceiling_kernel(const bf16x8* __restrict__ ops, int64_t iters,
                                                              float* __restrict__ out,
                                                              unsigned long long* __restrict__ clocks) {
  extern __shared__ char lds_pad[];  // sized by the host so that one workgroup holds a compute unit
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[gid * 8 + i];
    b[i] = ops[gid * 8 + 4 + i];
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
    if constexpr (ORDER == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + k) & 3], b[(k + 2 * j) & 3], acc[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (ORDER == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + k) & 3], b[(k + 2 * j) & 3], acc[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (ORDER == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + 2 * j + (j >> 2)) & 3], acc[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (ORDER == 3) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], acc[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // order 4: the same FLOP as 64 v_mfma_f32_16x16x32_bf16 (16x16 outputs,
      // K = 32) over 32 accumulators of 4 registers (the same 128 registers)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          f32x4 c = {acc[j >> 1][4 * (j & 1) + 0], acc[j >> 1][4 * (j & 1) + 1], acc[j >> 1][4 * (j & 1) + 2],
                     acc[j >> 1][4 * (j & 1) + 3]};
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(j + k) & 3], b[(k + 2 * j) & 3], c, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j >> 1][4 * (j & 1) + r] = c[r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[gid] = s;
  if (threadIdx.x == 0) {
    clocks[blockIdx.x * 4 + 0] = t0;
    clocks[blockIdx.x * 4 + 1] = t1;
    clocks[blockIdx.x * 4 + 2] = r0;
    clocks[blockIdx.x * 4 + 3] = r1;
  }
}

}  // namespace

extern "C" {

int flce_ceiling_mfma(const void* ops, int order, int64_t iters, int grid, int threads, int lds_bytes, float* out,
                      unsigned long long* clocks, void* stream) {
  if (!ops || !out || !clocks || grid < 1 || iters < 1 || order < 0 || order > 4) return -1;
  if (threads < 64 || threads > 512 || threads % 64 != 0 || lds_bytes < 0 || lds_bytes > 160 * 1024) return -1;
  if ((uintptr_t)ops % 16 != 0) return -1;
  hipStream_t s = (hipStream_t)stream;
  const void* fn[5] = {(const void*)flce_ceiling_kernel<0>, (const void*)flce_ceiling_kernel<1>,
                       (const void*)flce_ceiling_kernel<2>, (const void*)flce_ceiling_kernel<3>,
                       (const void*)flce_ceiling_kernel<4>};
  if (lds_bytes > 64 * 1024 &&
      hipFuncSetAttribute(fn[order], hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess)
    return -3;
  const bf16x8* o = (const bf16x8*)ops;
  switch (order) {
    case 0: hipLaunchKernelGGL((flce_ceiling_kernel<0>), dim3(grid), dim3(threads), lds_bytes, s, o, iters, out, clocks); break;
    case 1: hipLaunchKernelGGL((flce_ceiling_kernel<1>), dim3(grid), dim3(threads), lds_bytes, s, o, iters, out, clocks); break;
    case 2: hipLaunchKernelGGL((flce_ceiling_kernel<2>), dim3(grid), dim3(threads), lds_bytes, s, o, iters, out, clocks); break;
    case 3: hipLaunchKernelGGL((flce_ceiling_kernel<3>), dim3(grid), dim3(threads), lds_bytes, s, o, iters, out, clocks); break;
    default: hipLaunchKernelGGL((flce_ceiling_kernel<4>), dim3(grid), dim3(threads), lds_bytes, s, o, iters, out, clocks); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
