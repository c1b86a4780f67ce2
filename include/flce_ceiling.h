/*
 * flce_ceiling.h -- a measuring instrument beside libflce: the sustained
 * rate of the bf16 matrix-core instruction the forward's contraction runs on
 * (v_mfma_f32_32x32x16_bf16, 32x32 outputs, K = 16, fp32 accumulation), with
 * operands in registers and no memory traffic, on AMD Instinct MI355X
 * (gfx950). The logits of the page "Een gefuseerde forward-kernel voor
 * lineaire cross-entropy op Apple-GPU's" (section 1) are that contraction, so
 * this rate bounds the forward on the same part. Built as libflce_ceiling.so.
 */
#ifndef FLCE_CEILING_H
#define FLCE_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launch `grid` workgroups of `threads` threads (a multiple of 64, at most
 * 512) with `lds_bytes` of unused dynamic LDS (to hold one workgroup per
 * compute unit). Each thread loads 8 16-byte operand fragments (bf16x8) from
 * ops[(global thread index) * 8 + 0..7] -- ops must hold grid * threads * 8
 * such fragments, 16-byte aligned -- then runs `iters` iterations of 32
 * MFMAs over 8 accumulators:
 *   order 0: consecutive instructions write different accumulators and
 *            differ in both operands;
 *   order 1: each accumulator takes 4 instructions back to back;
 *   order 2: as 0, with the A operand held for 8 consecutive instructions;
 *   order 3: as 0, with both operands held for 8 consecutive instructions;
 *   order 4: the same FLOP as 64 v_mfma_f32_16x16x32_bf16 per iteration (16x16
 *            outputs, K = 32) over 32 accumulators of 4 registers, operands
 *            varied as in order 0.
 * FLOP per launch = grid * (threads / 64) * iters * 32 * 32768 (every order).
 * out (float32, grid * threads) receives each thread's accumulator sum, so
 * the work cannot be removed. clocks (uint64, grid * 4) receives, per
 * workgroup, s_memtime before and after the loop, then s_memrealtime (a
 * 100 MHz reference) before and after.
 * All pointers are device memory owned by the caller; stream is a
 * hipStream_t (NULL: default). Returns 0, -1 for a bad argument (nothing
 * enqueued) or -3 for a launch failure. Asynchronous on the stream.
 */
int flce_ceiling_mfma(const void* ops, int order, int64_t iters, int grid, int threads, int lds_bytes, float* out,
                      unsigned long long* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_CEILING_H */
