// C ABI of libsage.so: argument checking on the host, then the launches.
// Every check runs before anything is queued, so a rejected call touches no
// buffer and no device state, and the error paths run without a GPU.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/sage_probe.h"
#include "sage_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

// Device memory of sage_quantize_noalloc: the K-mean partial sums live here
// instead of in a caller's workspace.  One copy per GPU, resident until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, in noalloc_scratch() below.
constexpr size_t kScratchBytes = SAGE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call per device), or nullptr with the HIP error in *err.
void* noalloc_scratch(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Validates the shape; fills d.  Returns SAGE_OK or an error code.
int check_shape(const sage_shape* s, sage::Dims& d) {
    if (s == nullptr) return SAGE_EINVAL;
    if (s->B < 0 || s->H < 0 || s->N < 0) return SAGE_EINVAL;
    if (s->causal < 0 || s->causal > 1 || s->k_smooth < 0 || s->k_smooth > 1 || s->q_smooth < 0 ||
        s->q_smooth > 1 || s->dp_int8 < 0 || s->dp_int8 > 1 || s->p_static < 0 || s->p_static > 1 ||
        s->qk_norm < 0 || s->qk_norm > 1 || s->fp8 < 0 || s->fp8 > 1)
        return SAGE_EINVAL;
    if (s->fp8 && (s->dp_int8 || s->p_static)) return SAGE_EUNSUPPORTED;
    if (!(s->sm_scale >= 0.f) || !std::isfinite(s->sm_scale)) return SAGE_EINVAL;
    if (s->D != 64 && s->D != 128) return SAGE_EUNSUPPORTED;
    if (s->bq != 64 && s->bq != 128) return SAGE_EUNSUPPORTED;
    if (s->bkv != 64) return SAGE_EUNSUPPORTED;
    if (s->dtype != SAGE_FP16 && s->dtype != SAGE_BF16) return SAGE_EUNSUPPORTED;
    if (s->N % s->bq != 0 || s->N % s->bkv != 0) return SAGE_EUNSUPPORTED;
    // in-head offsets are 32-bit (16-bit element count fits), heads go on grid.y
    if ((int64_t)s->N * s->D * 2 > INT32_MAX) return SAGE_EUNSUPPORTED;
    if ((int64_t)s->B * s->H > 65535) return SAGE_EUNSUPPORTED;
    d.B = s->B; d.H = s->H; d.N = s->N; d.D = s->D; d.bq = s->bq; d.bkv = s->bkv;
    d.bf16 = s->dtype == SAGE_BF16;
    d.causal = s->causal != 0;
    d.k_smooth = s->k_smooth != 0;
    d.q_smooth = s->q_smooth != 0;
    d.dp_int8 = s->dp_int8 != 0;
    d.p_static = s->p_static != 0;
    d.qk_norm = s->qk_norm != 0;
    d.fp8 = s->fp8 != 0;
    d.scale = s->sm_scale > 0.f ? (double)s->sm_scale : 1.0 / std::sqrt((double)s->D);
    return SAGE_OK;
}

bool empty(const sage::Dims& d) { return d.B == 0 || d.H == 0 || d.N == 0; }

// Every listed pointer non-NULL and 16-byte aligned.
template <typename... P>
bool ptrs_ok(P... p) {
    const void* ps[] = {static_cast<const void*>(p)...};
    for (const void* x : ps)
        if (x == nullptr || !aligned(x, 16)) return false;
    return true;
}

int check_qtensors(const sage::Dims& d, const sage_qtensors* t) {
    if (t == nullptr) return SAGE_EINVAL;
    if (!ptrs_ok(t->q, t->sq, t->k, t->sk, t->vt, t->sv)) return SAGE_EINVAL;
    if (d.dp_int8 && !ptrs_ok(t->vr)) return SAGE_EINVAL;
    if (d.k_smooth && !ptrs_ok(t->mu_k)) return SAGE_EINVAL;
    if (d.q_smooth && !ptrs_ok(t->mu_q, t->qk_bias)) return SAGE_EINVAL;
    if (d.qk_norm && !ptrs_ok(t->rq, t->rk)) return SAGE_EINVAL;
    return SAGE_OK;
}

int check_dotensors(const sage::Dims& d, const sage_dotensors* t) {
    if (t == nullptr) return SAGE_EINVAL;
    if (!ptrs_ok(t->delta, t->dot, t->sdo)) return SAGE_EINVAL;
    if (d.dp_int8 && !ptrs_ok(t->dor)) return SAGE_EINVAL;
    return SAGE_OK;
}

int finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return SAGE_EHIP;
    }
    return SAGE_OK;
}

}  // namespace

extern "C" {

size_t sage_quantize_workspace_bytes(const sage_shape* shape) {
    sage::Dims d;
    if (check_shape(shape, d) != SAGE_OK) return 0;
    return (size_t)d.B * d.H * d.Tn() * d.D * sizeof(double);
}

int sage_quantize(const sage_shape* shape, const void* Q, const void* K, const void* V,
                  const sage_qtensors* out, void* workspace, sage_stream_t stream) {
    sage::Dims d;
    int st = check_shape(shape, d);
    if (st != SAGE_OK) return st;
    if (empty(d)) return SAGE_OK;
    if (!ptrs_ok(Q, K, V)) return SAGE_EINVAL;
    if ((st = check_qtensors(d, out)) != SAGE_OK) return st;
    if (d.k_smooth && (workspace == nullptr || !aligned(workspace, 8))) return SAGE_EINVAL;
    return finish(sage::launch_quantize(d, Q, K, V, *out, static_cast<double*>(workspace),
                                        reinterpret_cast<hipStream_t>(stream)));
}

int sage_quantize_noalloc(const sage_shape* shape, const void* Q, const void* K, const void* V,
                          const sage_qtensors* out, sage_stream_t stream) {
    sage::Dims d;
    int st = check_shape(shape, d);
    if (st != SAGE_OK) return st;
    if (empty(d)) return SAGE_OK;
    if (!ptrs_ok(Q, K, V)) return SAGE_EINVAL;
    if ((st = check_qtensors(d, out)) != SAGE_OK) return st;
    if (d.k_smooth && sage_quantize_workspace_bytes(shape) > kScratchBytes) return SAGE_ESCRATCH;
    hipError_t e = hipSuccess;
    void* ws = noalloc_scratch(&e);
    if (ws == nullptr) return finish(e);
    return finish(sage::launch_quantize(d, Q, K, V, *out, static_cast<double*>(ws),
                                        reinterpret_cast<hipStream_t>(stream)));
}

int sage_fwd(const sage_shape* shape, const sage_qtensors* qk, void* O, float* L, sage_stream_t stream) {
    sage::Dims d;
    int st = check_shape(shape, d);
    if (st != SAGE_OK) return st;
    if (empty(d)) return SAGE_OK;
    if ((st = check_qtensors(d, qk)) != SAGE_OK) return st;
    if (!ptrs_ok(O, L)) return SAGE_EINVAL;
    return finish(sage::launch_fwd(d, *qk, O, L, reinterpret_cast<hipStream_t>(stream)));
}

int sage_bwd_pre(const sage_shape* shape, const void* O, const void* dO, const sage_dotensors* out,
                 sage_stream_t stream) {
    sage::Dims d;
    int st = check_shape(shape, d);
    if (st != SAGE_OK) return st;
    if (empty(d)) return SAGE_OK;
    if (!ptrs_ok(O, dO)) return SAGE_EINVAL;
    if ((st = check_dotensors(d, out)) != SAGE_OK) return st;
    return finish(sage::launch_bwd_pre(d, O, dO, *out, reinterpret_cast<hipStream_t>(stream)));
}

size_t sage_bwd_workspace_bytes(const sage_shape* shape) {
    sage::Dims d;
    if (check_shape(shape, d) != SAGE_OK) return 0;
    return sage::bwd_workspace_bytes(d);
}

int sage_bwd(const sage_shape* shape, const sage_qtensors* qk, const sage_dotensors* dos, const void* V,
             const void* dO, const float* L, void* workspace, float* dQ, float* dK, float* dV,
             sage_stream_t stream) {
    sage::Dims d;
    int st = check_shape(shape, d);
    if (st != SAGE_OK) return st;
    if (empty(d)) return SAGE_OK;
    if ((st = check_qtensors(d, qk)) != SAGE_OK) return st;
    if ((st = check_dotensors(d, dos)) != SAGE_OK) return st;
    if (!ptrs_ok(V, dO, L, workspace, dQ, dK, dV)) return SAGE_EINVAL;
    return finish(sage::launch_bwd(d, *qk, *dos, V, dO, L, workspace, dQ, dK, dV,
                                   reinterpret_cast<hipStream_t>(stream)));
}

int sage_qk_norm_bwd(const sage_shape* shape, const void* Q, const void* K, const sage_qtensors* qk, float* dQ,
                     float* dK, sage_stream_t stream) {
    sage::Dims d;
    int st = check_shape(shape, d);
    if (st != SAGE_OK) return st;
    if (!d.qk_norm || qk == nullptr) return SAGE_EINVAL;
    if (empty(d)) return SAGE_OK;
    if (!ptrs_ok(Q, K, qk->rq, qk->rk, dQ, dK)) return SAGE_EINVAL;
    return finish(sage::launch_qk_norm_bwd(d, Q, K, qk->rq, qk->rk, dQ, dK, reinterpret_cast<hipStream_t>(stream)));
}

int sage_cast_grads(const sage_shape* shape, const float* dQ, const float* dK, const float* dV, void* dQ16,
                    void* dK16, void* dV16, sage_stream_t stream) {
    sage::Dims d;
    int st = check_shape(shape, d);
    if (st != SAGE_OK) return st;
    const float* src[3] = {dQ, dK, dV};
    void* dst[3] = {dQ16, dK16, dV16};
    for (int t = 0; t < 3; ++t) {
        if ((src[t] == nullptr) != (dst[t] == nullptr)) return SAGE_EINVAL;
        if (src[t] != nullptr && !ptrs_ok(src[t], dst[t])) return SAGE_EINVAL;
    }
    if (empty(d) || (dQ == nullptr && dK == nullptr && dV == nullptr)) return SAGE_OK;
    return finish(sage::launch_cast_grads(d, src, dst, reinterpret_cast<hipStream_t>(stream)));
}

const char* sage_status_str(int status) {
    switch (status) {
        case SAGE_OK: return "ok";
        case SAGE_EINVAL: return "invalid argument (NULL or misaligned pointer, negative size, bad flag)";
        case SAGE_EUNSUPPORTED: return "unsupported shape (D, block sizes, dtype, or N not a multiple of the blocks)";
        case SAGE_EHIP: return "HIP launch failed (see sage_last_hip_error)";
        case SAGE_ESCRATCH:
            return "problem too large for the no-alloc entry point's fixed device scratch "
                   "(use sage_quantize with a workspace)";
        default: return "unknown status";
    }
}

int sage_last_hip_error(void) { return g_last_hip_error; }

int sage_probe_mfma_i8(int blocks, int iters, unsigned long long* clk, hipStream_t stream) {
    if (blocks < 1 || iters < 1 || clk == nullptr || !aligned(clk, 8)) return SAGE_EINVAL;
    return finish(sage::launch_probe_mfma_i8(blocks, iters, clk, stream));
}

int sage_probe_mfma_bf16(int blocks, int iters, unsigned long long* clk, hipStream_t stream) {
    if (blocks < 1 || iters < 1 || clk == nullptr || !aligned(clk, 8)) return SAGE_EINVAL;
    return finish(sage::launch_probe_mfma_bf16(blocks, iters, clk, stream));
}

int sage_probe_fp8_products(const int8_t* a, const int8_t* b, float* c32, float* c128, hipStream_t stream) {
    if (!ptrs_ok(a, b, c32, c128)) return SAGE_EINVAL;
    return finish(sage::launch_probe_fp8_products(a, b, c32, c128, stream));
}

const char* sage_version(void) { return "sage-mi355x 0.1 (gfx950)"; }

}  // extern "C"
