// Measurement aid: the achieved rate of the INT8 16x16x64 matrix product and
// the shader clock under that load (declared in include/sage_probe.h).
#include "sage_device.h"
#include "sage_internal.h"

namespace sage {
namespace {

constexpr int kChains = 8;   // independent accumulations per wave

__global__ __launch_bounds__(512, 2) void probe_mfma_i8_kernel(int iters, unsigned long long* clk) {
    const int lane = threadIdx.x & 63;
    const v4i a = v4i{lane, lane + 1, lane + 2, lane + 3};
    const v4i b = v4i{3 * lane, lane ^ 5, lane + 7, 11};
    v4i acc[kChains];
#pragma unroll
    for (int u = 0; u < kChains; ++u) acc[u] = v4i{u, 0, 0, 0};
    const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
    unsigned long long t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_readcyclecounter();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kChains; ++u) acc[u] = mfma16_i8(a, b, acc[u]);
    }
    int s = 0;
#pragma unroll
    for (int u = 0; u < kChains; ++u) s += acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3];
    if (s == 0x13572468) clk[2] = (unsigned long long)s;   // keeps the products live
    if (timer) {
        clk[0] = __builtin_readcyclecounter() - t0;
        clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

}  // namespace

hipError_t launch_probe_mfma_i8(int blocks, int iters, unsigned long long* clk, hipStream_t stream) {
    probe_mfma_i8_kernel<<<dim3(blocks), dim3(512), 0, stream>>>(iters, clk);
    return hipGetLastError();
}

}  // namespace sage
