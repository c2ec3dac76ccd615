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

#ifdef __cplusplus
extern "C" {
#endif

int sage_probe_mfma_i8(int blocks, int iters, unsigned long long* clk, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_PROBE_H */
