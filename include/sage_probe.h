/*
 * sage_probe.h — a measurement aid exported by libsage.so beside the
 * attention calls of sage.h (it computes nothing of the method).
 *
 * sage_probe_mfma_i8 runs `blocks` workgroups of 512 threads (8 waves), each
 * wave issuing `iters` rounds of 8 independent v_mfma_i32_16x16x64_i8
 * products (32 768 integer operations each) on register operands, so that
 * the achieved INT8 matrix rate of the device can be measured beside the
 * published 5.0 POP/s: time the call on `stream` (e.g. with events) and
 * divide blocks * 8 * iters * 8 * 32768 operations by the elapsed time.
 *
 *   clk   device pointer to 3 uint64_t, 8-byte aligned, written by the call:
 *         clk[0] = shader clock cycles and clk[1] = ticks of the constant
 *         100 MHz counter elapsed in workgroup 0's first lane (their ratio
 *         times 100 MHz is the shader clock under this load); clk[2] is
 *         scratch.  Owned by the caller.
 *   Returns 0 (SAGE_OK), SAGE_EINVAL for blocks < 1, iters < 1 or a NULL or
 *   misaligned clk (nothing launched), or SAGE_EHIP if the launch failed.
 *   Asynchronous on `stream`.
 */
#ifndef SAGE_PROBE_H
#define SAGE_PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int sage_probe_mfma_i8(int blocks, int iters, unsigned long long* clk, hipStream_t stream);

/*
 * sage_probe_mfma_bf16 is the same measurement on the BF16 matrix product
 * the backward's dP = dO V^T runs on: each wave issues `iters` rounds of 8
 * independent v_mfma_f32_16x16x32_bf16 products (16 384 floating-point
 * operations each) on register operands, beside the published 2.5 PFLOP/s
 * dense BF16 figure.  Divide blocks * 8 * iters * 8 * 16384 operations by the
 * elapsed time.  clk, return values and errors as for sage_probe_mfma_i8.
 */
int sage_probe_mfma_bf16(int blocks, int iters, unsigned long long* clk, hipStream_t stream);

/*
 * sage_probe_fp8_products runs one wave of the two E4M3 matrix products the
 * E4M3 variant uses (sage_shape.fp8), so that their lane layout and their
 * summation can be checked against exact products:
 *   a, b  device pointers, 64 * 32 bytes each (16-byte aligned): lane l's 32
 *         E4M3 bytes at offset 32 l.  Lane l supplies row l % 16 of A and
 *         column l % 16 of B; in v_mfma_f32_16x16x32_fp8_fp8 its first 8
 *         bytes carry contraction indices 8 (l / 16) + e, and in
 *         v_mfma_f32_16x16x128_f8f6f4 (E4M3, no block scale) all 32 bytes
 *         carry 32 (l / 16) + e.
 *   c32, c128  device pointers, 64 * 4 floats each: lane l's result
 *         registers j = 0..3 (row 4 (l / 16) + j, column l % 16) of each
 *         product, accumulated from zero.  Owned by the caller.
 *   Returns 0, SAGE_EINVAL for a NULL or misaligned pointer (nothing
 *   launched), or SAGE_EHIP.  Asynchronous on `stream`.
 */
int sage_probe_fp8_products(const int8_t* a, const int8_t* b, float* c32, float* c128, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_PROBE_H */
