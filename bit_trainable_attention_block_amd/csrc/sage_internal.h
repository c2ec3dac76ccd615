// Host-side declarations shared by the translation units of libsage.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sage.h"

namespace sage {

// Validated, derived view of a sage_shape.
struct Dims {
    int B, H, N, D, bq, bkv;
    bool bf16, causal, k_smooth, q_smooth;
    bool dp_int8;  // ablation: dP from the INT8 codes of dO and V
    bool p_static; // ablation: static forward P scale 1/127
    bool qk_norm;  // QK-norm fused into the preprocessing
    bool fp8;      // variant: E4M3 codes, 448 in place of 127
    double scale;  // softmax scale; 1/sqrt(D) in double unless given
    int BH() const { return B * H; }
    int Tm() const { return N / bq; }
    int Tn() const { return N / bkv; }
    size_t head_elems() const { return (size_t)N * D; }
};

// Launchers; each returns hipSuccess or the launch error.
hipError_t launch_quantize(const Dims& d, const void* Q, const void* K, const void* V,
                           const sage_qtensors& out, double* ws, hipStream_t s);
hipError_t launch_bwd_pre(const Dims& d, const void* O, const void* dO, const sage_dotensors& out,
                          hipStream_t s);
hipError_t launch_fwd(const Dims& d, const sage_qtensors& qk, void* O, float* L, hipStream_t s);
size_t bwd_workspace_bytes(const Dims& d);
hipError_t launch_bwd(const Dims& d, const sage_qtensors& qk, const sage_dotensors& dos, const void* V,
                      const void* dO, const float* L, void* workspace, float* dQ, float* dK, float* dV,
                      hipStream_t s);
hipError_t launch_qk_norm_bwd(const Dims& d, const void* Q, const void* K, const float* rq, const float* rk,
                              float* dQ, float* dK, hipStream_t s);
hipError_t launch_cast_grads(const Dims& d, const float* const src[3], void* const dst[3], hipStream_t s);
hipError_t launch_probe_mfma_i8(int blocks, int iters, unsigned long long* clk, hipStream_t s);
hipError_t launch_probe_mfma_bf16(int blocks, int iters, unsigned long long* clk, hipStream_t s);
hipError_t launch_probe_fp8_products(const int8_t* a, const int8_t* b, float* c32, float* c128,
                                     hipStream_t stream);

}  // namespace sage
