// Preprocessing kernels of the SageBwd path: K/Q smoothing, per-block INT8
// quantisation of Q, K, V (SageBwd method summary, forward steps (1)-(2);
// SageAttention3 write-up Eq. 7) and the backward pre-pass
// D = rowsum(dO o O) plus dO quantisation (backward step (1)).
//
// All of it is HBM-bound streaming: each workgroup owns one quantisation
// block (64 or 128 rows x D columns of one head), reads it once with 16-byte
// loads, reduces max|x| in registers / DPP / LDS, and writes the INT8 codes in
// the operand layouts the attention kernels consume (see sage.h), staged
// through LDS so every global store is a coalesced 16-byte store.
//
// Codes and scales must equal the definition bit for bit:
//   s = f32(max|x| / 127) with a correctly rounded division, and
//   code = clamp(rint(f32(x / s)), -127, 127), ties to even;
// in the E4M3 variant s = f32(max|x| / 448) and the code is the nearest E4M3
// value of f32(x / s), ties to even (v_cvt_pk_fp8_f32 rounds that way).
// Hence __fdiv_rn / __fsub_rn, the exact float64 form of f32(x / s) in
// codes_to_lds, and no fast-math anywhere in this file.
#include "sage_device.h"
#include "sage_internal.h"

namespace sage {
namespace {

constexpr int kThreads = 256;

template <int R, int D>
struct Blk {
    static constexpr int CPR = D / 8;                 // 16-byte input chunks per row
    static constexpr int PER_T = R * CPR / kThreads;  // chunks per thread
    static constexpr int RSTEP = kThreads / CPR;      // rows between a thread's chunks
    static_assert(PER_T >= 1 && R * CPR % kThreads == 0, "block shape");
};

// Load a block of 16-bit values: thread t gets the chunks (row, cc) with
// cc = t % CPR and rows t / CPR + k * RSTEP.
template <int R, int D>
__device__ __forceinline__ void load_block(const u16* __restrict__ src, v4i (&raw)[Blk<R, D>::PER_T]) {
    using B = Blk<R, D>;
    const int t = threadIdx.x;
    const int cc = t % B::CPR;
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k) {
        int row = t / B::CPR + k * B::RSTEP;
        raw[k] = *reinterpret_cast<const v4i*>(src + (size_t)row * D + cc * 8);
    }
}

template <bool BF16>
__device__ __forceinline__ void unpack8(v4i r, float (&x)[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t u = (uint32_t)r[w];
        x[2 * w] = to_f32<BF16>((u16)(u & 0xffff));
        x[2 * w + 1] = to_f32<BF16>((u16)(u >> 16));
    }
}

__device__ __forceinline__ float block_max(float m, float* red) {
    m = wave_max(m);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = m;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

// Column sums in float64 over the thread's rows, reduced across the RSTEP
// threads sharing a column chunk; result for column c in dsum[c].
// red holds kThreads rows of 9 doubles (8 sums and a pad, so that the
// column reads below fall on distinct LDS banks).
constexpr int kRedStride = 9;

template <int R, int D>
__device__ __forceinline__ void block_colsum(const double (&part)[8], double* red, double* dsum) {
    using B = Blk<R, D>;
    const int t = threadIdx.x;
#pragma unroll
    for (int c = 0; c < 8; ++c) red[t * kRedStride + c] = part[c];
    __syncthreads();
    if (t < D) {
        const int cc = t / 8, c = t % 8;
        double s = 0.0;
        for (int r = 0; r < B::RSTEP; ++r) s += red[(r * B::CPR + cc) * kRedStride + c];
        dsum[t] = s;
    }
    __syncthreads();
}

// QK-norm of the block's rows in place (unit gain): per row
//   r = f32(1 / sqrt(mean(x^2) + eps))    (sum of squares exact in float64,
//                                          then IEEE double sqrt and divide)
//   x = f32(x * r)                         (one rounding; no contraction)
// The CPR threads of a row are consecutive lanes, so the row sum is a lane
// reduction.  r of each row goes to rout[row0 + row] when rout is set.
constexpr double kQkNormEps = 1e-6;

template <int R, int D>
using BlockVals = float[Blk<R, D>::PER_T][8];

template <int R, int D>
__device__ __forceinline__ void rms_normalize(BlockVals<R, D>& x, float* __restrict__ rout, int row0) {
    using B = Blk<R, D>;
    const int t = threadIdx.x;
    const int cc = t % B::CPR;
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k) {
        double ss = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (double)x[k][e] * (double)x[k][e];
        ss = wave_sum_d(ss, B::CPR);
        const float r = (float)__ddiv_rn(1.0, __dsqrt_rn(ss / (double)D + kQkNormEps));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[k][e] = __fmul_rn(x[k][e], r);
        if (rout != nullptr && cc == 0) rout[row0 + t / B::CPR + k * B::RSTEP] = r;
    }
}

// Row stride of the LDS code buffers: 16 bytes of padding per row, so the
// R32 gather (16-byte chunks of consecutive rows in consecutive lanes) steps
// through the LDS banks instead of hitting every row at the same bank.
template <int D>
constexpr int CStride = D + 16;

// Largest code magnitude: INT8 or E4M3.
__device__ __forceinline__ float qmax_of(int fp8) { return fp8 ? 448.f : 127.f; }

// Quantise x (values of the block held per thread) with scale s and store
// the codes (INT8, or E4M3 bytes) row-major into LDS codes[R][CStride<D>].
template <int R, int D>
__device__ __forceinline__ void codes_to_lds(const float (&x)[Blk<R, D>::PER_T][8], float s,
                                             uint8_t* codes, int fp8) {
    using B = Blk<R, D>;
    const int t = threadIdx.x;
    const int cc = t % B::CPR;
    // x / s correctly rounded to float32 without a division per element.
    // With r = RN64(1/s) (one division per block), RN64(x r) lies within
    // 2^-52 (relative) of x / s.  A quotient of two float32 values is never
    // within 2^-49 of a float32 rounding midpoint: a midpoint m has 25
    // significant bits, so x - m s is a nonzero multiple of a power of two no
    // smaller than 2^-49 |x|.  Rounding RN64(x r) to float32 is therefore
    // RN32(x / s) exactly.  A zero block (s = 0) gets r = 0 and zero codes.
    const double r = s > 0.f ? __ddiv_rn(1.0, (double)s) : 0.0;
    auto quot = [r](float v) __attribute__((always_inline)) {
        return __double2float_rn(__dmul_rn((double)v, r));
    };
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k) {
        int row = t / B::CPR + k * B::RSTEP;
        uint2 w;
        if (fp8) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = quot(x[k][e]);
            w.x = (uint32_t)pack_e4m3(v[0], v[1], v[2], v[3]);
            w.y = (uint32_t)pack_e4m3(v[4], v[5], v[6], v[7]);
        } else {
            int c[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = code_i8(quot(x[k][e]));
            w.x = pack4(c[0], c[1], c[2], c[3]);
            w.y = pack4(c[4], c[5], c[6], c[7]);
        }
        *reinterpret_cast<uint2*>(codes + row * CStride<D> + cc * 8) = w;
    }
}

enum Layout { R32, C64P };

// In-block row of byte e of output chunk g for the C64P column layout.
__device__ __forceinline__ int c64p_row(int grp_part, int e) { return 16 * (e >> 2) + 4 * grp_part + (e & 3); }

// Write the R x D codes held in LDS to dst (the block's region of the head,
// laid out as L) with coalesced 16-byte stores.
template <Layout L, int R, int D>
__device__ __forceinline__ void store_codes(const uint8_t* codes, int8_t* __restrict__ dst) {
    constexpr int CHUNKS = R * D / 16;
    for (int oc = threadIdx.x; oc < CHUNKS; oc += kThreads) {
        v4i out;
        if constexpr (L == R32) {
            const int g = oc / (2 * D), rem = oc % (2 * D);
            const int col16 = rem / 32, r = rem % 32;
            out = *reinterpret_cast<const v4i*>(codes + (32 * g + r) * CStride<D> + col16 * 16);
        } else {
            constexpr int GR = 64;                     // rows per group
            constexpr int PARTS = GR / 16;             // h or g values
            const int grp = oc / (PARTS * D), rem = oc % (PARTS * D);
            const int part = rem / D, col = rem % D;
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t acc = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int row = grp * GR + c64p_row(part, 4 * q + b);
                    acc |= (uint32_t)codes[row * CStride<D> + col] << (8 * b);
                }
                w[q] = acc;
            }
            out = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
        *reinterpret_cast<v4i*>(dst + (size_t)oc * 16) = out;
    }
}

// ------------------------------------------------------------------ kernels

// V blocks (64 rows): codes -> vt (C64P), scale -> sv; with dp_int8 the
// codes again, as R32 row tiles, -> vr (the INT8-dP ablation's operand).
// K blocks (same rows): the block's float64 column sums -> kpart[bh][j][D]
// (a fixed summation order inside the block; kmean_kernel adds the blocks in
// order, so mu_K does not depend on scheduling even where the float64 sums
// round, as they can for the QK-normed float32 rows).
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void quant_v_ksum_kernel(
    const u16* __restrict__ K, const u16* __restrict__ V, int N, int8_t* __restrict__ vt,
    float* __restrict__ sv, int8_t* __restrict__ vr, double* __restrict__ kpart, int k_smooth, int dp_int8,
    int qk_norm, int fp8) {
    constexpr int R = 64;
    using B = Blk<R, D>;
    __shared__ float red[4];
    __shared__ __align__(16) uint8_t codes[R * CStride<D>];
    __shared__ double dred[kRedStride * kThreads];
    __shared__ double dsum[D];
    const int j = blockIdx.x, bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const int row0 = j * R;

    v4i raw[B::PER_T];
    float x[B::PER_T][8];
    load_block<R, D>(V + head + (size_t)row0 * D, raw);
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k) {
        unpack8<BF16>(raw[k], x[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[k][e]));
    }
    const float a = block_max(m, red);
    const float s = __fdiv_rn(a, qmax_of(fp8));
    codes_to_lds<R, D>(x, s, codes, fp8);
    if (threadIdx.x == 0) sv[(size_t)bh * (N / R) + j] = s;
    __syncthreads();
    store_codes<C64P, R, D>(codes, vt + head + (size_t)row0 * D);
    if (dp_int8) store_codes<R32, R, D>(codes, vr + head + (size_t)row0 * D);

    if (k_smooth) {
        load_block<R, D>(K + head + (size_t)row0 * D, raw);
        float y[B::PER_T][8];
#pragma unroll
        for (int k = 0; k < B::PER_T; ++k) unpack8<BF16>(raw[k], y[k]);
        if (qk_norm) rms_normalize<R, D>(y, nullptr, row0);   // the mean of the normalised rows
        double part[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < B::PER_T; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) part[e] += (double)y[k][e];
        block_colsum<R, D>(part, dred, dsum);
        if (threadIdx.x < D) kpart[((size_t)bh * gridDim.x + j) * D + threadIdx.x] = dsum[threadIdx.x];
    }
}

// mu_K[bh][c] = f32(sum_j kpart[bh][j][c] / N) in float64, in a fixed order:
// the Tn block sums of a head are split into G consecutive runs, thread
// (run, channel) adds its run in block order, and the G run sums are added in
// run order.  Reads are coalesced across the channels of a block.
template <int D>
__global__ __launch_bounds__(512) void kmean_kernel(const double* __restrict__ kpart, int Tn, int N,
                                                    float* __restrict__ mu_k) {
    constexpr int G = 512 / D;
    __shared__ double part[G][D];
    const int bh = blockIdx.x, c = threadIdx.x % D, run = threadIdx.x / D;
    const double* p = kpart + (size_t)bh * Tn * D + c;
    const int j0 = run * Tn / G, j1 = (run + 1) * Tn / G;
    double acc = 0.0;
#pragma unroll 8
    for (int j = j0; j < j1; ++j) acc += p[(size_t)j * D];
    part[run][c] = acc;
    __syncthreads();
    if (run == 0) {
        double sum = part[0][c];
#pragma unroll
        for (int r = 1; r < G; ++r) sum += part[r][c];
        mu_k[(size_t)bh * D + c] = (float)(sum / (double)N);
    }
}

// Q blocks (BQ rows): optional Q-smoothing (QS, mu_q set), codes -> q (R32).
// Only with QS does the block hold the column-sum scratch.
template <bool BF16, int D, int BQ, bool QS, bool QKN>
__global__ __launch_bounds__(kThreads) void quant_q_kernel(const u16* __restrict__ Q, int N,
                                                           int8_t* __restrict__ q,
                                                           float* __restrict__ sq,
                                                           float* __restrict__ mu_q,
                                                           float* __restrict__ rq, int fp8) {
    using B = Blk<BQ, D>;
    __shared__ float red[4];
    __shared__ __align__(16) uint8_t codes[BQ * CStride<D>];
    __shared__ double dred[QS ? kRedStride * kThreads : 1];
    __shared__ double dsum[QS ? D : 1];
    __shared__ float mu[QS ? D : 1];
    const int i = blockIdx.x, bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const int row0 = i * BQ;
    const int Tm = N / BQ;

    v4i raw[B::PER_T];
    float x[B::PER_T][8];
    load_block<BQ, D>(Q + head + (size_t)row0 * D, raw);
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k) unpack8<BF16>(raw[k], x[k]);
    if constexpr (QKN) rms_normalize<BQ, D>(x, rq + (size_t)bh * N, row0);

    if constexpr (QS) {
        double part[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < B::PER_T; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) part[e] += (double)x[k][e];
        block_colsum<BQ, D>(part, dred, dsum);
        if (threadIdx.x < D) {
            const float mv = (float)(dsum[threadIdx.x] / (double)BQ);
            mu[threadIdx.x] = mv;
            mu_q[((size_t)bh * Tm + i) * D + threadIdx.x] = mv;
        }
        __syncthreads();
        const int cc = threadIdx.x % B::CPR;
#pragma unroll
        for (int k = 0; k < B::PER_T; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[k][e] = __fsub_rn(x[k][e], mu[cc * 8 + e]);
    }
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[k][e]));
    const float a = block_max(m, red);
    const float s = __fdiv_rn(a, qmax_of(fp8));
    codes_to_lds<BQ, D>(x, s, codes, fp8);
    if (threadIdx.x == 0) sq[(size_t)bh * Tm + i] = s;
    __syncthreads();
    store_codes<R32, BQ, D>(codes, q + head + (size_t)row0 * D);
}

// K blocks (64 rows): K_sm = f32(K - mu_K) (mu_K from kmean_kernel); codes
// -> k (R32).  With Q-smoothing, also the logit bias of these keys
// for every query block that sees them: bias[i][n] = scale * sum_c mu_Q[i][c]
// * K_sm[n][c] (exact float64 products and float64 sums, rounded once).  QS:
// Q-smoothing on (qk_bias set); only then does the block hold its smoothed
// rows in LDS.
template <bool BF16, int D, bool QS>
__global__ __launch_bounds__(kThreads) void quant_k_kernel(
    const u16* __restrict__ K, int N, int8_t* __restrict__ k,
    float* __restrict__ sk, const float* __restrict__ mu_k, int k_smooth,
    const float* __restrict__ mu_q, float* __restrict__ qk_bias, int Tm, double scale, float* __restrict__ rk,
    int fp8, int causal) {
    constexpr int R = 64;
    using B = Blk<R, D>;
    __shared__ float red[4];
    __shared__ __align__(16) uint8_t codes[R * CStride<D>];
    __shared__ float mu[D];
    // K_sm rows; once each wave holds its keys' values in registers, the
    // same LDS takes two stages of a 16-row tile of mu_Q (Q-smoothing bias),
    // whose padding puts the A-operand reads (16 rows x 4 consecutive
    // channels per instruction) on 64 distinct banks
    constexpr int KSM_FLOATS = QS ? R * (D + 1) : 1;
    constexpr int MUQ_FLOATS = QS ? 2 * 16 * (D + 4) : 1;
    static_assert(MUQ_FLOATS <= KSM_FLOATS, "the mu_Q stages reuse the K_sm rows");
    __shared__ __align__(16) float ksm_raw[KSM_FLOATS];
    auto ksm = reinterpret_cast<float(*)[QS ? D + 1 : 1]>(ksm_raw);
    auto muq = reinterpret_cast<float(*)[16][QS ? D + 4 : 1]>(ksm_raw);
    const int j = blockIdx.x, bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const int row0 = j * R;

    // the block's rows are requested first; the mean arrives meanwhile
    v4i raw[B::PER_T];
    load_block<R, D>(K + head + (size_t)row0 * D, raw);
    if (threadIdx.x < D) mu[threadIdx.x] = k_smooth ? mu_k[(size_t)bh * D + threadIdx.x] : 0.f;
    __syncthreads();

    float x[B::PER_T][8];
    const int cc = threadIdx.x % B::CPR;
#pragma unroll
    for (int kk = 0; kk < B::PER_T; ++kk) unpack8<BF16>(raw[kk], x[kk]);
    if (rk != nullptr) rms_normalize<R, D>(x, rk + (size_t)bh * N, row0);
    float m = 0.f;
#pragma unroll
    for (int kk = 0; kk < B::PER_T; ++kk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (k_smooth) x[kk][e] = __fsub_rn(x[kk][e], mu[cc * 8 + e]);
            m = fmaxf(m, fabsf(x[kk][e]));
        }
    }
    const float a = block_max(m, red);
    const float s = __fdiv_rn(a, qmax_of(fp8));
    codes_to_lds<R, D>(x, s, codes, fp8);
    if (threadIdx.x == 0) sk[(size_t)bh * (N / R) + j] = s;
    if constexpr (QS) {
#pragma unroll
        for (int kk = 0; kk < B::PER_T; ++kk) {
            int row = threadIdx.x / B::CPR + kk * B::RSTEP;
#pragma unroll
            for (int e = 0; e < 8; ++e) ksm[row][cc * 8 + e] = x[kk][e];
        }
    }
    __syncthreads();
    store_codes<R32, R, D>(codes, k + head + (size_t)row0 * D);

    if constexpr (QS) {
        // The bias tile mu_Q (query blocks x D) . K_sm^T (D x the block's 64
        // keys) on the float64 matrix cores (v_mfma_f64_16x16x4_f64: exact
        // products, float64 sums).  Wave w owns keys 16 w .. 16 w + 15, whose
        // K_sm values stay in registers as the B operands of all D / 4
        // contraction steps (lane l: key 16 w + l % 16, channels 4 k + l / 16).
        // The workgroup walks the query blocks 16 at a time; each tile of mu_Q
        // rows goes through LDS (two stages, the next tile's coalesced loads
        // in flight during this tile's products) and gives the A operands
        // (lane l: query block i0 + l % 16, the same channels).  Result
        // register r of lane l is query block i0 + l / 16 + 4 r, key
        // 16 w + l % 16 (the float64 product's row order: rows interleave over
        // the lane groups).  Under causal masking only the query blocks from
        // the first one that sees a key of the block's 128-key pair on are
        // computed (the backward takes its key blocks in pairs from that
        // query block on); no kernel reads the others.
        constexpr int KS = D / 4;
        constexpr int TL = 16 * D / 4 / kThreads;   // float4 loads per thread per tile
        static_assert(TL >= 1 && 16 * D / 4 == TL * kThreads, "mu_Q tile shape");
        const int lane = threadIdx.x & 63;
        const int wq = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int cl = lane >> 4, rl = lane & 15;
        double bk[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) bk[kk] = (double)ksm[16 * wq + rl][4 * kk + cl];
        const int bq = N / Tm;
        const int i_first = causal ? ((row0 >> 7) << 7) / bq : 0;
        const int ntiles = (Tm - i_first + 15) / 16;
        typedef double v4d __attribute__((ext_vector_type(4)));
        const float* mqh = mu_q + (size_t)bh * Tm * D;
        // thread t's share of a tile: float4 number t + kThreads u, i.e. row
        // (t + kThreads u) / (D / 4), channels 4 ((t + kThreads u) % (D / 4))..
        auto fetch = [&](int i0, v4f (&buf)[TL]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < TL; ++u) {
                const int f = threadIdx.x + kThreads * u;
                const int row = i0 + f / (D / 4);
                buf[u] = row < Tm ? *reinterpret_cast<const v4f*>(mqh + (size_t)row * D + 4 * (f % (D / 4)))
                                  : v4f{0.f, 0.f, 0.f, 0.f};
            }
        };
        auto put = [&](int stage, const v4f (&buf)[TL]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < TL; ++u) {
                const int f = threadIdx.x + kThreads * u;
                *reinterpret_cast<v4f*>(&muq[stage][f / (D / 4)][4 * (f % (D / 4))]) = buf[u];
            }
        };
        v4f pre[TL];
        if (ntiles > 0) fetch(i_first, pre);
        __syncthreads();   // every wave holds its K_sm values: the rows' LDS takes the mu_Q stages
        if (ntiles > 0) put(0, pre);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            const int i0 = i_first + 16 * t;
            if (t + 1 < ntiles) fetch(i0 + 16, pre);
            // four independent accumulation chains over the contraction
            // steps (kk % 4), added at the end: the products of one chain
            // wait for each other, those of different chains do not
            v4d acc4[4];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) acc4[c4] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                acc4[kk & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)muq[t & 1][rl][4 * kk + cl], bk[kk],
                                                                     acc4[kk & 3], 0, 0, 0);
            const v4d acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + cl + 4 * r;
                if (i < Tm) qk_bias[((size_t)bh * Tm + i) * N + row0 + 16 * wq + rl] = (float)(acc[r] * scale);
            }
            if (t + 1 < ntiles) put((t + 1) & 1, pre);
            __syncthreads();   // the next tile is in LDS; this one may be overwritten
        }
    }
}

// Backward pre-pass on one BQ-row block: delta = rowsum(dO o O) (float64,
// rounded once), dO codes -> dot (C64P), scale -> sdo; with dp_int8 the codes
// again, as R32 row tiles, -> dor (the INT8-dP ablation's operand).
template <bool BF16, int D, int BQ>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const u16* __restrict__ O,
                                                           const u16* __restrict__ dO, int N,
                                                           float* __restrict__ delta,
                                                           int8_t* __restrict__ dot,
                                                           float* __restrict__ sdo,
                                                           int8_t* __restrict__ dor, int dp_int8, int fp8) {
    using B = Blk<BQ, D>;
    __shared__ float red[4];
    __shared__ __align__(16) uint8_t codes[BQ * CStride<D>];
    const int i = blockIdx.x, bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const int row0 = i * BQ;
    const int Tm = N / BQ;
    const int cc = threadIdx.x % B::CPR;

    v4i raw[B::PER_T], rawo[B::PER_T];
    float x[B::PER_T][8];
    load_block<BQ, D>(dO + head + (size_t)row0 * D, raw);
    load_block<BQ, D>(O + head + (size_t)row0 * D, rawo);
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k) {
        float o[8];
        unpack8<BF16>(raw[k], x[k]);
        unpack8<BF16>(rawo[k], o);
        double acc = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc += (double)x[k][e] * (double)o[e];
            m = fmaxf(m, fabsf(x[k][e]));
        }
        // the CPR threads of a row are consecutive lanes of one wave
        acc = wave_sum_d(acc, B::CPR);
        if (cc == 0) delta[(size_t)bh * N + row0 + threadIdx.x / B::CPR + k * B::RSTEP] = (float)acc;
    }
    const float a = block_max(m, red);
    const float s = __fdiv_rn(a, qmax_of(fp8));
    codes_to_lds<BQ, D>(x, s, codes, fp8);
    if (threadIdx.x == 0) sdo[(size_t)bh * Tm + i] = s;
    __syncthreads();
    store_codes<C64P, BQ, D>(codes, dot + head + (size_t)row0 * D);
    if (dp_int8) store_codes<R32, BQ, D>(codes, dor + head + (size_t)row0 * D);
}

// Gradient through QK-norm, in place on one 64-row block of one head:
//   x_n = f32(x * r) (as the forward formed it), c = mean(dX_n o x_n)
//   (float64), dX = r * (dX_n - x_n * c).
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void qk_norm_bwd_kernel(const u16* __restrict__ X, const float* __restrict__ r,
                                                               float* __restrict__ dX, int N) {
    constexpr int R = 64;
    using B = Blk<R, D>;
    const int j = blockIdx.x, bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const int row0 = j * R;
    const int t = threadIdx.x, cc = t % B::CPR;
    v4i raw[B::PER_T];
    load_block<R, D>(X + head + (size_t)row0 * D, raw);
#pragma unroll
    for (int k = 0; k < B::PER_T; ++k) {
        const int row = row0 + t / B::CPR + k * B::RSTEP;
        float x[8];
        unpack8<BF16>(raw[k], x);
        const float rr = r[(size_t)bh * N + row];
        float* g = dX + head + (size_t)row * D + cc * 8;
        const v4f g0 = *reinterpret_cast<const v4f*>(g), g1 = *reinterpret_cast<const v4f*>(g + 4);
        const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        float xn[8];
        double c = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            xn[e] = __fmul_rn(x[e], rr);
            c += (double)gv[e] * (double)xn[e];
        }
        c = wave_sum_d(c, B::CPR) / (double)D;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (float)((double)rr * ((double)gv[e] - (double)xn[e] * c));
        *reinterpret_cast<v4f*>(g) = v4f{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<v4f*>(g + 4) = v4f{o[4], o[5], o[6], o[7]};
    }
}

template <bool BF16, int D>
hipError_t quantize_impl(const Dims& d, const void* Q, const void* K, const void* V,
                         const sage_qtensors& out, double* ws, hipStream_t s) {
    const int BH = d.BH();
    dim3 blk(kThreads);
    quant_v_ksum_kernel<BF16, D><<<dim3(d.Tn(), BH), blk, 0, s>>>(
        (const u16*)K, (const u16*)V, d.N, out.vt, out.sv, out.vr, ws, d.k_smooth ? 1 : 0, d.dp_int8 ? 1 : 0,
        d.qk_norm ? 1 : 0, d.fp8 ? 1 : 0);
    if (d.k_smooth) kmean_kernel<D><<<dim3(BH), dim3(512), 0, s>>>(ws, d.Tn(), d.N, out.mu_k);
    // fused QK-norm as a template switch: its float64 row sums would
    // otherwise set the register count (and the occupancy) of every launch
    auto qq = d.qk_norm ? (d.bq == 128 ? (d.q_smooth ? quant_q_kernel<BF16, D, 128, true, true>
                                                    : quant_q_kernel<BF16, D, 128, false, true>)
                                       : (d.q_smooth ? quant_q_kernel<BF16, D, 64, true, true>
                                                     : quant_q_kernel<BF16, D, 64, false, true>))
                        : (d.bq == 128 ? (d.q_smooth ? quant_q_kernel<BF16, D, 128, true, false>
                                                    : quant_q_kernel<BF16, D, 128, false, false>)
                                       : (d.q_smooth ? quant_q_kernel<BF16, D, 64, true, false>
                                                     : quant_q_kernel<BF16, D, 64, false, false>));
    qq<<<dim3(d.Tm(), BH), blk, 0, s>>>((const u16*)Q, d.N, out.q, out.sq, d.q_smooth ? out.mu_q : nullptr,
                                        d.qk_norm ? out.rq : nullptr, d.fp8 ? 1 : 0);
    auto kq = d.q_smooth ? quant_k_kernel<BF16, D, true> : quant_k_kernel<BF16, D, false>;
    kq<<<dim3(d.Tn(), BH), blk, 0, s>>>(
        (const u16*)K, d.N, out.k, out.sk, out.mu_k, d.k_smooth ? 1 : 0,
        d.q_smooth ? out.mu_q : nullptr, d.q_smooth ? out.qk_bias : nullptr, d.Tm(), d.scale,
        d.qk_norm ? out.rk : nullptr, d.fp8 ? 1 : 0, d.causal ? 1 : 0);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t bwd_pre_impl(const Dims& d, const void* O, const void* dO, const sage_dotensors& out,
                        hipStream_t s) {
    dim3 grid(d.Tm(), d.BH());
    if (d.bq == 128)
        bwd_pre_kernel<BF16, D, 128><<<grid, kThreads, 0, s>>>((const u16*)O, (const u16*)dO, d.N,
                                                               out.delta, out.dot, out.sdo, out.dor,
                                                               d.dp_int8 ? 1 : 0, d.fp8 ? 1 : 0);
    else
        bwd_pre_kernel<BF16, D, 64><<<grid, kThreads, 0, s>>>((const u16*)O, (const u16*)dO, d.N,
                                                              out.delta, out.dot, out.sdo, out.dor,
                                                              d.dp_int8 ? 1 : 0, d.fp8 ? 1 : 0);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t qk_norm_bwd_impl(const Dims& d, const void* Q, const void* K, const float* rq, const float* rk,
                            float* dQ, float* dK, hipStream_t s) {
    const dim3 grid(d.N / 64, d.BH());
    qk_norm_bwd_kernel<BF16, D><<<grid, kThreads, 0, s>>>((const u16*)Q, rq, dQ, d.N);
    qk_norm_bwd_kernel<BF16, D><<<grid, kThreads, 0, s>>>((const u16*)K, rk, dK, d.N);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm_bwd(const Dims& d, const void* Q, const void* K, const float* rq, const float* rk,
                              float* dQ, float* dK, hipStream_t s) {
    if (d.bf16)
        return d.D == 128 ? qk_norm_bwd_impl<true, 128>(d, Q, K, rq, rk, dQ, dK, s)
                          : qk_norm_bwd_impl<true, 64>(d, Q, K, rq, rk, dQ, dK, s);
    return d.D == 128 ? qk_norm_bwd_impl<false, 128>(d, Q, K, rq, rk, dQ, dK, s)
                      : qk_norm_bwd_impl<false, 64>(d, Q, K, rq, rk, dQ, dK, s);
}

hipError_t launch_quantize(const Dims& d, const void* Q, const void* K, const void* V,
                           const sage_qtensors& out, double* ws, hipStream_t s) {
    if (d.bf16) {
        return d.D == 128 ? quantize_impl<true, 128>(d, Q, K, V, out, ws, s)
                          : quantize_impl<true, 64>(d, Q, K, V, out, ws, s);
    }
    return d.D == 128 ? quantize_impl<false, 128>(d, Q, K, V, out, ws, s)
                      : quantize_impl<false, 64>(d, Q, K, V, out, ws, s);
}

hipError_t launch_bwd_pre(const Dims& d, const void* O, const void* dO, const sage_dotensors& out,
                          hipStream_t s) {
    if (d.bf16) {
        return d.D == 128 ? bwd_pre_impl<true, 128>(d, O, dO, out, s) : bwd_pre_impl<true, 64>(d, O, dO, out, s);
    }
    return d.D == 128 ? bwd_pre_impl<false, 128>(d, O, dO, out, s) : bwd_pre_impl<false, 64>(d, O, dO, out, s);
}


namespace {

// Eight float32 gradient elements per thread -> eight 16-bit values (two
// 16-byte loads, one 16-byte store); tensor t = blockIdx.y.  n8 = elements / 8.
struct CastArgs {
    const float* src[3];
    u16* dst[3];
};

template <bool BF16>
__global__ __launch_bounds__(256) void cast_grads_kernel(CastArgs a, size_t n8) {
    const float* src = a.src[blockIdx.y];
    u16* dst = a.dst[blockIdx.y];
    if (src == nullptr) return;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (size_t)gridDim.x * blockDim.x) {
        const float4 lo = reinterpret_cast<const float4*>(src)[2 * i];
        const float4 hi = reinterpret_cast<const float4*>(src)[2 * i + 1];
        const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        v4i out;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[e] = (int)((uint32_t)from_f32<BF16>(x[2 * e]) | ((uint32_t)from_f32<BF16>(x[2 * e + 1]) << 16));
        reinterpret_cast<v4i*>(dst)[i] = out;
    }
}

}  // namespace

hipError_t launch_cast_grads(const Dims& d, const float* const src[3], void* const dst[3], hipStream_t s) {
    CastArgs a;
    for (int t = 0; t < 3; ++t) {
        a.src[t] = src[t];
        a.dst[t] = static_cast<u16*>(dst[t]);
    }
    const size_t n8 = (size_t)d.BH() * d.head_elems() / 8;   // D is 64 or 128: whole groups of eight
    const size_t want = (n8 + 255) / 256;
    const dim3 grid((unsigned)(want < 8192 ? want : 8192), 3);
    if (d.bf16) cast_grads_kernel<true><<<grid, 256, 0, s>>>(a, n8);
    else cast_grads_kernel<false><<<grid, 256, 0, s>>>(a, n8);
    return hipGetLastError();
}

}  // namespace sage
