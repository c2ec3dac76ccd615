// SageBwd INT8 backward (SageBwd method summary, backward steps (2)-(7);
// SageAttention3 write-up Eq. 9 and its INT8 updates), key blocks outer and
// query blocks inner (paperlayer appendix A.1), in two kernels:
//
// 1. bwd_kernel — one workgroup = 8 waves = two 64-key blocks of one head;
//    wave w owns 16 keys of block 2*jj + w/4 and keeps their dV and dK in
//    float32 registers for the whole sweep over query tiles.  Per query tile
//    (BQ rows, the dO/Q quantisation block) the Q codes, dO (16-bit), the
//    transposed Q and dO codes and the per-row L and delta are staged in LDS
//    once for both key blocks, and each wave computes, on the matrix cores
//    (16x16 tiles, lane = key):
//      S  = Q^ K^T     v_mfma_i32_16x16x64_i8            (recompute)
//      dP = dO V^T     v_mfma_f32_16x16x32_{bf16,f16}    (kept in 16-bit)
//    then on the vector units P = 2^(S log2e - L log2e), dS = P (dP - delta);
//    the per-tile maxima of P and |dS| (one scale per BQ x 64 tile) go
//    through LDS once, and the codes feed, straight from registers,
//      dV^T += dO^^T P^   and   dK^T += Q^^T dS^        (16x16x64 i8)
//    because S's result order is the operand order once the transposed codes
//    are stored permuted (C64P).  The dS codes of each tile (BQ x 64 bytes)
//    and its scale go to the workspace, already in the dQ product's operand
//    order.
// 2. dq_kernel — one workgroup per query tile: dQ_i = sum_j dS^_ij K^_j
//    s_dS,ij s_K,j (INT8 products, int32 per tile, float32 across tiles),
//    written once: no atomics and no clearing pass.
//
// Codes are rounded to nearest-even by one fma with 1.5 * 2^23, which leaves
// the integer in the low mantissa byte, and packed with v_perm.
#include <algorithm>

#include "sage_device.h"
#include "sage_internal.h"

namespace sage {
namespace {

struct BwdArgs {
    const int8_t* q;
    const int8_t* qt;
    const float* sq;
    const int8_t* k;
    const int8_t* kt;
    const float* sk;
    const u16* vr;
    const float* mu_q;
    const float* qk_bias;
    const float* delta;
    const int8_t* dot;
    const float* sdo;
    const u16* dor;
    const float* L;
    int8_t* dsw;   // dS codes per tile, [bh][tile][4][BQ][16]
    float* sds;    // dS scale per tile, [bh][tile]
    float* dQ;
    float* dK;
    float* dV;
    int N;
    double scale;  // softmax scale
};

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

// Tiles per head and the index of tile (i, j) in the workspace; causal heads
// store only the visible tiles, row i holding j < (i + 1) * BQ / 64.
template <int BQ, bool CAUSAL>
__host__ __device__ __forceinline__ size_t tiles_per_head(int Tm, int Tn) {
    constexpr int R = BQ / 64;
    return CAUSAL ? (size_t)R * Tm * (Tm + 1) / 2 : (size_t)Tm * Tn;
}
template <int BQ, bool CAUSAL>
__device__ __forceinline__ size_t tile_index(int i, int j, int Tn) {
    constexpr int R = BQ / 64;
    return CAUSAL ? (size_t)R * i * (i + 1) / 2 + j : (size_t)i * Tn + j;
}

// Byte 0 of four magic-rounded floats -> one dword (rows r = 0..3).
__device__ __forceinline__ int pack_magic(float a, float b, float c, float d) {
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x04000c0cu);
    return (int)(lo | hi);
}

template <int BQ, int D>
struct BwdSmem {
    int8_t q[BQ * D];            // Q codes, R32
    int8_t qt[BQ * D];           // Q codes, C64P
    int8_t dot[BQ * D];          // dO codes, C64P
    u16 dor[BQ * D];             // dO, R16H
    int8_t ds[2][4 * BQ * 16];   // dS codes of the two key blocks, [key/16][query][16]
    float l2[BQ];                // L * log2 e
    float delta[BQ];
    float red[2][2][4];          // [key block][P | dS][wave]
    float sds[2];                // dS scale of the two key blocks
};

template <bool BF16, int D, int BQ, bool CAUSAL, bool QSMOOTH>
__global__ __launch_bounds__(512, 1) void bwd_kernel(BwdArgs a) {
    constexpr int NT = 512;
    constexpr int MB = BQ / 16;   // 16-query blocks per tile
    constexpr int KQ = BQ / 64;   // i8 contraction steps over queries
    constexpr int KS8 = D / 64;   // i8 contraction steps over d
    constexpr int KSH = D / 32;   // 16-bit contraction steps over d
    constexpr int DB = D / 16;    // 16-wide blocks of d
    __shared__ __align__(16) BwdSmem<BQ, D> sm;

    const int N = a.N;
    const int Tn = N / 64, Tm = N / BQ;
    const int jj = blockIdx.x, bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
    const int kb = w >> 2, kg = w & 3;
    const int j = 2 * jj + kb;        // this wave's key block
    const bool kv_on = j < Tn;        // the second block of a ragged tail may not exist
    const int key = j * 64 + 16 * kg + n16;

    v4i kop[KS8], vop[KSH];
    float skj = 0.f;
    if (kv_on) {
#pragma unroll
        for (int ks = 0; ks < KS8; ++ks)
            kop[ks] = *reinterpret_cast<const v4i*>(a.k + head + off_r32(key, 64 * ks + 16 * g, D));
#pragma unroll
        for (int ks = 0; ks < KSH; ++ks)
            vop[ks] = *reinterpret_cast<const v4i*>(a.vr + head + off_r16h(key, 32 * ks + 8 * g, D));
        skj = a.sk[(size_t)bh * Tn + j];
    }

    v4f dvt[DB], dkt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dvt[db] = v4f{0, 0, 0, 0};
        dkt[db] = v4f{0, 0, 0, 0};
    }

    const size_t tph = tiles_per_head<BQ, CAUSAL>(Tm, Tn);
    const int istart = CAUSAL ? (2 * jj * 64) / BQ : 0;
    for (int i = istart; i < Tm; ++i) {
        const int qbase = i * BQ;
        // ---- stage the query tile (read by the waves of both key blocks)
        {
            const v4i* src_q = reinterpret_cast<const v4i*>(a.q + head + (size_t)qbase * D);
            const v4i* src_qt = reinterpret_cast<const v4i*>(a.qt + head + (size_t)qbase * D);
            const v4i* src_dot = reinterpret_cast<const v4i*>(a.dot + head + (size_t)qbase * D);
            const v4i* src_dor = reinterpret_cast<const v4i*>(a.dor + head + (size_t)qbase * D);
            v4i* dq_ = reinterpret_cast<v4i*>(sm.q);
            v4i* dqt = reinterpret_cast<v4i*>(sm.qt);
            v4i* ddot = reinterpret_cast<v4i*>(sm.dot);
            v4i* ddor = reinterpret_cast<v4i*>(sm.dor);
#pragma unroll
            for (int c = tid; c < BQ * D / 16; c += NT) {
                dq_[c] = src_q[c];
                dqt[c] = src_qt[c];
                ddot[c] = src_dot[c];
            }
#pragma unroll
            for (int c = tid; c < BQ * D / 8; c += NT) ddor[c] = src_dor[c];
            if (tid < BQ) {
                sm.l2[tid] = (float)((double)a.L[(size_t)bh * N + qbase + tid] * kLog2e_d);
                sm.delta[tid] = a.delta[(size_t)bh * N + qbase + tid];
            }
        }
        __syncthreads();

        const bool tile_on = kv_on && (!CAUSAL || j * 64 <= qbase + BQ - 1);
        const float sqi = a.sq[(size_t)bh * Tm + i];
        float p[MB][4], ds[MB][4];
        float pmax = 0.f, dsmax = 0.f;
        if (tile_on) {
            const float c2 = (float)((double)sqi * (double)skj * a.scale * kLog2e_d);  // one rounding
            float bias2 = 0.f;
            if (QSMOOTH) bias2 = (float)((double)a.qk_bias[((size_t)bh * Tm + i) * N + key] * kLog2e_d);
            const bool need_mask = CAUSAL && (j * 64 + 63 > qbase);
            // ---- S and dP for this wave's 16 keys and all BQ queries
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = 16 * mb + n16;  // query row (in tile) this lane supplies
                v4i s = v4i{0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS8; ++ks) {
                    const v4i av = *reinterpret_cast<const v4i*>(sm.q + off_r32(row, 64 * ks + 16 * g, D));
                    s = mfma16_i8(av, kop[ks], s);
                }
                v4f dp = v4f{0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KSH; ++ks) {
                    const v4i av = *reinterpret_cast<const v4i*>(sm.dor + off_r16h(row, 32 * ks + 8 * g, D));
                    dp = mfma16_h<BF16>(av, vop[ks], dp);
                }
                const v4f l2 = *reinterpret_cast<const v4f*>(&sm.l2[16 * mb + 4 * g]);
                const v4f dl = *reinterpret_cast<const v4f*>(&sm.delta[16 * mb + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = fmaf((float)s[r], c2, -l2[r]);
                    if (QSMOOTH) x += bias2;
                    float pv = __builtin_amdgcn_exp2f(x);
                    if (need_mask && key > qbase + 16 * mb + 4 * g + r) pv = 0.f;
                    const float dsv = pv * (dp[r] - dl[r]);
                    p[mb][r] = pv;
                    ds[mb][r] = dsv;
                    pmax = fmaxf(pmax, pv);
                    dsmax = fmaxf(dsmax, fabsf(dsv));
                }
            }
        }
        // ---- per-tile maxima over the key block's four waves
        pmax = wave_max(pmax);
        dsmax = wave_max(dsmax);
        if (lane == 0) {
            sm.red[kb][0][kg] = pmax;
            sm.red[kb][1][kg] = dsmax;
        }
        __syncthreads();
        pmax = fmaxf(fmaxf(sm.red[kb][0][0], sm.red[kb][0][1]), fmaxf(sm.red[kb][0][2], sm.red[kb][0][3]));
        dsmax = fmaxf(fmaxf(sm.red[kb][1][0], sm.red[kb][1][1]), fmaxf(sm.red[kb][1][2], sm.red[kb][1][3]));
        const float sP = __fdiv_rn(pmax, 127.f);
        const float sS = __fdiv_rn(dsmax, 127.f);
        if (tid == 256 * kb) sm.sds[kb] = sS;

        if (tile_on) {
            const float invP = sP > 0.f ? 1.f / sP : 0.f;
            const float invS = sS > 0.f ? 1.f / sS : 0.f;
            // ---- codes; dS codes also to LDS (query on the lane, for dQ)
            v4i pop[KQ], dsop[KQ];
            int8_t* dsl = sm.ds[kb] + kg * BQ * 16;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float pc[4], sc[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pc[r] = fmaf(p[mb][r], invP, kMagic);  // rint(P / s_P) in the low byte
                    sc[r] = fmaf(ds[mb][r], invS, kMagic);
                }
                pop[mb >> 2][mb & 3] = pack_magic(pc[0], pc[1], pc[2], pc[3]);
                const int sw = pack_magic(sc[0], sc[1], sc[2], sc[3]);
                dsop[mb >> 2][mb & 3] = sw;
#pragma unroll
                for (int r = 0; r < 4; ++r) dsl[(16 * mb + 4 * g + r) * 16 + n16] = (int8_t)(sw >> (8 * r));
            }
            if (QSMOOTH) {
                // dK bias (dS^T 1) mu_Q^T from the unquantised dS
                float cs = 0.f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) cs += ds[mb][r];
                cs += __shfl_xor(cs, 16);
                cs += __shfl_xor(cs, 32);
                const float* mq = a.mu_q + ((size_t)bh * Tm + i) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const v4f m4 = *reinterpret_cast<const v4f*>(mq + 16 * db + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dkt[db][r] = fmaf(cs, m4[r], dkt[db][r]);
                }
            }
            // ---- dV^T += dO^^T P^,  dK^T += Q^^T dS^
            const float fv = sP * a.sdo[(size_t)bh * Tm + i];
            const float fk = sS * sqi;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                v4i accv = v4i{0, 0, 0, 0}, acck = v4i{0, 0, 0, 0};
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) {
                    const int chunk = kq * 4 * D + g * D + 16 * db + n16;
                    const v4i av = reinterpret_cast<const v4i*>(sm.dot)[chunk];
                    const v4i ak = reinterpret_cast<const v4i*>(sm.qt)[chunk];
                    accv = mfma16_i8(av, pop[kq], accv);
                    acck = mfma16_i8(ak, dsop[kq], acck);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dvt[db][r] = fmaf((float)accv[r], fv, dvt[db][r]);
                    dkt[db][r] = fmaf((float)acck[r], fk, dkt[db][r]);
                }
            }
        }
        __syncthreads();  // dS tiles complete in LDS; the staged tile is no longer read

        // ---- dS codes and scales of the visible tiles to the workspace
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            const int jb = 2 * jj + b2;
            if (jb < Tn && (!CAUSAL || jb * 64 <= qbase + BQ - 1)) {
                const size_t t = (size_t)bh * tph + tile_index<BQ, CAUSAL>(i, jb, Tn);
                const v4i* src = reinterpret_cast<const v4i*>(sm.ds[b2]);
                v4i* dst = reinterpret_cast<v4i*>(a.dsw + t * (BQ * 64));
                for (int c = tid; c < BQ * 64 / 16; c += NT) dst[c] = src[c];
                if (tid == 0) a.sds[t] = sm.sds[b2];
            }
        }
        __syncthreads();  // LDS reused by the next tile
    }

    // ---- write dV and dK (lane = key, 4 consecutive d per block)
    if (kv_on) {
        float* dV = a.dV + head + (size_t)key * D;
        float* dK = a.dK + head + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            v4f kv;
#pragma unroll
            for (int r = 0; r < 4; ++r) kv[r] = (float)((double)dkt[db][r] * a.scale);
            *reinterpret_cast<v4f*>(dV + 16 * db + 4 * g) = dvt[db];
            *reinterpret_cast<v4f*>(dK + 16 * db + 4 * g) = kv;
        }
    }
}

// dQ_i = scale * sum_j s_dS,ij s_K,j M(dS^_ij, K^_j), one workgroup per query
// tile; wave w owns BQ/4 queries and all D columns.
template <int D, int BQ, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void dq_kernel(const int8_t* __restrict__ dsw, const float* __restrict__ sds,
                                                   const int8_t* __restrict__ kt, const float* __restrict__ sk,
                                                   float* __restrict__ dQ, int N, double scale) {
    constexpr int QPW = BQ / 4;           // queries per wave
    constexpr int MBq = QPW / 16;
    constexpr int NB = D / 16;
    constexpr int DS_BYTES = BQ * 64;
    constexpr int K_BYTES = 64 * D;
    constexpr int CH = (DS_BYTES + K_BYTES) / 16;   // 16-byte chunks per stage
    constexpr int CPT = (CH + 255) / 256;
    __shared__ __align__(16) int8_t stage[2][DS_BYTES + K_BYTES];

    const int Tn = N / 64, Tm = N / BQ;
    const int i = CAUSAL ? (Tm - 1 - (int)blockIdx.x) : (int)blockIdx.x;  // heavy tiles first
    const int bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const size_t tph = tiles_per_head<BQ, CAUSAL>(Tm, Tn);
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
    const int jend = CAUSAL ? (i + 1) * BQ / 64 : Tn;

    auto load = [&](int j, v4i (&buf)[CPT]) {
        const size_t t = (size_t)bh * tph + tile_index<BQ, CAUSAL>(i, j, Tn);
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = tid + u * 256;
            if (c < DS_BYTES / 16)
                buf[u] = reinterpret_cast<const v4i*>(dsw + t * DS_BYTES)[c];
            else if (c < CH)
                buf[u] = reinterpret_cast<const v4i*>(kt + head + (size_t)j * K_BYTES)[c - DS_BYTES / 16];
        }
    };
    auto store = [&](int sidx, const v4i (&buf)[CPT]) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = tid + u * 256;
            if (c < CH) reinterpret_cast<v4i*>(stage[sidx])[c] = buf[u];
        }
    };

    v4f acc[MBq][NB];
#pragma unroll
    for (int mb = 0; mb < MBq; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = v4f{0, 0, 0, 0};

    v4i pre[CPT];
    load(0, pre);
    store(0, pre);
    __syncthreads();
    for (int j = 0; j < jend; ++j) {
        const int sidx = j & 1;
        const bool more = j + 1 < jend;
        if (more) load(j + 1, pre);
        const size_t t = (size_t)bh * tph + tile_index<BQ, CAUSAL>(i, j, Tn);
        const float cj = (float)((double)sds[t] * (double)sk[(size_t)bh * Tn + j] * scale);
        const v4i* lds = reinterpret_cast<const v4i*>(stage[sidx]);
        const v4i* lk = reinterpret_cast<const v4i*>(stage[sidx] + DS_BYTES);
        v4i av[MBq];
#pragma unroll
        for (int mb = 0; mb < MBq; ++mb) av[mb] = lds[g * BQ + QPW * w + 16 * mb + n16];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const v4i bv = lk[g * D + 16 * nb + n16];
#pragma unroll
            for (int mb = 0; mb < MBq; ++mb) {
                const v4i x = mfma16_i8(av[mb], bv, v4i{0, 0, 0, 0});
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mb][nb][r] = fmaf((float)x[r], cj, acc[mb][nb][r]);
            }
        }
        if (more) {
            __syncthreads();
            store(sidx ^ 1, pre);
            __syncthreads();
        }
    }
    float* out = dQ + head + (size_t)(i * BQ + QPW * w) * D;
#pragma unroll
    for (int mb = 0; mb < MBq; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[(size_t)(16 * mb + 4 * g + r) * D + 16 * nb + n16] = acc[mb][nb][r];
}

template <bool BF16, int D, int BQ, bool CAUSAL>
hipError_t bwd_dispatch(const Dims& d, const BwdArgs& a, hipStream_t s) {
    const dim3 grid((d.Tn() + 1) / 2, d.BH());
    if (d.q_smooth) bwd_kernel<BF16, D, BQ, CAUSAL, true><<<grid, 512, 0, s>>>(a);
    else bwd_kernel<BF16, D, BQ, CAUSAL, false><<<grid, 512, 0, s>>>(a);
    dq_kernel<D, BQ, CAUSAL><<<dim3(d.Tm(), d.BH()), 256, 0, s>>>(a.dsw, a.sds, a.kt, a.sk, a.dQ, d.N, d.scale);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t bwd_dispatch_bq(const Dims& d, const BwdArgs& a, hipStream_t s) {
    if (d.bq == 128)
        return d.causal ? bwd_dispatch<BF16, D, 128, true>(d, a, s) : bwd_dispatch<BF16, D, 128, false>(d, a, s);
    return d.causal ? bwd_dispatch<BF16, D, 64, true>(d, a, s) : bwd_dispatch<BF16, D, 64, false>(d, a, s);
}

size_t total_tiles(const Dims& d) {
    if (d.bq == 128)
        return d.BH() * (d.causal ? tiles_per_head<128, true>(d.Tm(), d.Tn()) : tiles_per_head<128, false>(d.Tm(), d.Tn()));
    return d.BH() * (d.causal ? tiles_per_head<64, true>(d.Tm(), d.Tn()) : tiles_per_head<64, false>(d.Tm(), d.Tn()));
}

size_t codes_bytes(const Dims& d) { return (total_tiles(d) * (size_t)d.bq * 64 + 255) / 256 * 256; }

}  // namespace

size_t bwd_workspace_bytes(const Dims& d) { return codes_bytes(d) + total_tiles(d) * sizeof(float); }

hipError_t launch_bwd(const Dims& d, const sage_qtensors& qk, const sage_dotensors& dos, const float* L,
                      void* workspace, float* dQ, float* dK, float* dV, hipStream_t s) {
    int8_t* dsw = static_cast<int8_t*>(workspace);
    float* sds = reinterpret_cast<float*>(dsw + codes_bytes(d));
    const BwdArgs a{qk.q,  qk.qt, qk.sq, qk.k, qk.kt, qk.sk, qk.vr, qk.mu_q, qk.qk_bias, dos.delta, dos.dot,
                    dos.sdo, dos.dor, L, dsw, sds, dQ, dK, dV, d.N, d.scale};
    if (d.bf16) return d.D == 128 ? bwd_dispatch_bq<true, 128>(d, a, s) : bwd_dispatch_bq<true, 64>(d, a, s);
    return d.D == 128 ? bwd_dispatch_bq<false, 128>(d, a, s) : bwd_dispatch_bq<false, 64>(d, a, s);
}

}  // namespace sage
