// SageBwd INT8 backward (SageBwd method summary, backward steps (2)-(7);
// SageAttention3 write-up Eq. 9 and its INT8 updates), key blocks outer and
// query blocks inner (paperlayer appendix A.1).
//
// One workgroup = 4 waves = one 64-key block of one head; wave w owns keys
// 16w..16w+15 and keeps their dV and dK in float32 registers for the whole
// sweep over query tiles.  Per query tile (BQ rows, the dO/Q quantisation
// block) the Q codes, dO (16-bit), the transposed Q and dO codes and the
// per-row L and delta are staged in LDS, and each wave computes, on the
// matrix cores (16x16 tiles, lane = key):
//   S   = Q^ K^T       v_mfma_i32_16x16x64_i8      (recompute)
//   dP  = dO V^T       v_mfma_f32_16x16x32_{bf16,f16}   (kept in 16-bit)
// then on the vector units P = 2^(S log2e - L log2e), dS = P (dP - delta);
// the per-tile maxima of P and |dS| (one scale per BQ x 64 tile) go through
// LDS once, and the codes feed, straight from registers,
//   dV^T += dO^^T P^   and   dK^T += Q^^T dS^      (16x16x64 i8)
// because S's result order is the operand order once the transposed codes
// are stored permuted (C64P).  dQ = dS^ K^ needs dS^ with the query on the
// lane, so the dS codes make one trip through LDS; the four waves then split
// dQ's columns and add their float32 results with hardware atomics.
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
    float* dQ;
    float* dK;
    float* dV;
    int N;
    double scale;   // softmax scale
};

template <int BQ, int D>
struct BwdSmem {
    int8_t q[BQ * D];        // Q codes, R32
    int8_t qt[BQ * D];       // Q codes, C64P
    int8_t dot[BQ * D];      // dO codes, C64P
    u16 dor[BQ * D];         // dO, R16H
    int8_t ds[4 * BQ * 16];  // dS codes, [key/16][query][16]
    float l2[BQ];            // L * log2 e
    float delta[BQ];
    float red[2][4];
};

template <bool BF16, int D, int BQ, bool CAUSAL, bool QSMOOTH>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdArgs a) {
    constexpr int MB = BQ / 16;   // 16-query blocks per tile
    constexpr int KS8 = D / 64;   // i8 contraction steps over d
    constexpr int KSH = D / 32;   // 16-bit contraction steps over d
    constexpr int DB = D / 16;    // 16-wide blocks of d
    constexpr int KQ = BQ / 64;   // i8 contraction steps over queries
    constexpr int NB = D / 64;    // dQ column blocks per wave (D/4 columns)
    __shared__ __align__(16) BwdSmem<BQ, D> sm;

    const int N = a.N;
    const int Tn = N / 64, Tm = N / BQ;
    const int j = blockIdx.x, bh = blockIdx.y;
    const size_t head = (size_t)bh * N * D;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
    const int key = j * 64 + 16 * w + n16;

    // Loop-invariant B operands of this wave's 16 keys.
    v4i kop[KS8];
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks)
        kop[ks] = *reinterpret_cast<const v4i*>(a.k + head + off_r32(key, 64 * ks + 16 * g, D));
    v4i vop[KSH];
#pragma unroll
    for (int ks = 0; ks < KSH; ++ks)
        vop[ks] = *reinterpret_cast<const v4i*>(a.vr + head + off_r16h(key, 32 * ks + 8 * g, D));
    // K codes with keys on the contraction index, for dQ (columns of this wave)
    v4i ktop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int dcol = (D / 4) * w + 16 * nb + n16;
        ktop[nb] = *reinterpret_cast<const v4i*>(a.kt + head + (size_t)j * 64 * D + (g * D + dcol) * 16);
    }
    const float skj = a.sk[(size_t)bh * Tn + j];

    v4f dvt[DB], dkt[DB], dkb[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dvt[db] = v4f{0, 0, 0, 0};
        dkt[db] = v4f{0, 0, 0, 0};
        dkb[db] = v4f{0, 0, 0, 0};
    }

    const int istart = CAUSAL ? (j * 64) / BQ : 0;
    for (int i = istart; i < Tm; ++i) {
        const int qbase = i * BQ;
        // ---- stage the query tile
        {
            const v4i* src_q = reinterpret_cast<const v4i*>(a.q + head + (size_t)qbase * D);
            const v4i* src_qt = reinterpret_cast<const v4i*>(a.qt + head + (size_t)qbase * D);
            const v4i* src_dot = reinterpret_cast<const v4i*>(a.dot + head + (size_t)qbase * D);
            const v4i* src_dor = reinterpret_cast<const v4i*>(a.dor + head + (size_t)qbase * D);
            v4i* dq_ = reinterpret_cast<v4i*>(sm.q);
            v4i* dqt = reinterpret_cast<v4i*>(sm.qt);
            v4i* ddot = reinterpret_cast<v4i*>(sm.dot);
            v4i* ddor = reinterpret_cast<v4i*>(sm.dor);
            for (int c = tid; c < BQ * D / 16; c += 256) {
                dq_[c] = src_q[c];
                dqt[c] = src_qt[c];
                ddot[c] = src_dot[c];
            }
            for (int c = tid; c < BQ * D / 8; c += 256) ddor[c] = src_dor[c];
            if (tid < BQ) {
                sm.l2[tid] = (float)((double)a.L[(size_t)bh * N + qbase + tid] * kLog2e_d);
                sm.delta[tid] = a.delta[(size_t)bh * N + qbase + tid];
            }
        }
        __syncthreads();

        const float sqi = a.sq[(size_t)bh * Tm + i];
        const float c2 = (float)((double)sqi * (double)skj * a.scale * kLog2e_d);  // one rounding
        float bias2 = 0.f;
        if (QSMOOTH) bias2 = (float)((double)a.qk_bias[((size_t)bh * Tm + i) * N + key] * kLog2e_d);
        const bool need_mask = CAUSAL && (j * 64 + 63 > qbase);

        // ---- S and dP for this wave's 16 keys and all BQ queries
        float p[MB][4], ds[MB][4];
        float pmax = 0.f, dsmax = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = 16 * mb + n16;  // query row (in tile) this lane supplies
            v4i s = v4i{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS8; ++ks) {
                v4i av = *reinterpret_cast<const v4i*>(sm.q + off_r32(row, 64 * ks + 16 * g, D));
                s = mfma16_i8(av, kop[ks], s);
            }
            v4f dp = v4f{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KSH; ++ks) {
                v4i av = *reinterpret_cast<const v4i*>(sm.dor + off_r16h(row, 32 * ks + 8 * g, D));
                dp = mfma16_h<BF16>(av, vop[ks], dp);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ql = 16 * mb + 4 * g + r;  // query (in tile) of result register r
                float x = fmaf((float)s[r], c2, -sm.l2[ql]);
                if (QSMOOTH) x += bias2;
                float pv = exp2f(x);
                if (need_mask && key > qbase + ql) pv = 0.f;
                const float dsv = pv * (dp[r] - sm.delta[ql]);
                p[mb][r] = pv;
                ds[mb][r] = dsv;
                pmax = fmaxf(pmax, pv);
                dsmax = fmaxf(dsmax, fabsf(dsv));
            }
        }
        pmax = wave_max(pmax);
        dsmax = wave_max(dsmax);
        if (lane == 0) {
            sm.red[0][w] = pmax;
            sm.red[1][w] = dsmax;
        }
        __syncthreads();
        pmax = fmaxf(fmaxf(sm.red[0][0], sm.red[0][1]), fmaxf(sm.red[0][2], sm.red[0][3]));
        dsmax = fmaxf(fmaxf(sm.red[1][0], sm.red[1][1]), fmaxf(sm.red[1][2], sm.red[1][3]));
        const float sP = __fdiv_rn(pmax, 127.f);
        const float sS = __fdiv_rn(dsmax, 127.f);
        const float invP = sP > 0.f ? 1.f / sP : 0.f;
        const float invS = sS > 0.f ? 1.f / sS : 0.f;

        // ---- codes; dS codes also to LDS (query on the lane for dQ)
        v4i pop[KQ], dsop[KQ];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            int pc[4], sc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pc[r] = (int)rintf(p[mb][r] * invP);
                sc[r] = code_i8(ds[mb][r] * invS);
                sm.ds[(w * BQ + 16 * mb + 4 * g + r) * 16 + n16] = (int8_t)sc[r];
            }
            pop[mb >> 2][mb & 3] = (int)pack4(pc[0], pc[1], pc[2], pc[3]);
            dsop[mb >> 2][mb & 3] = (int)pack4(sc[0], sc[1], sc[2], sc[3]);
        }
        if (QSMOOTH) {
            float cs = 0.f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) cs += ds[mb][r];
            cs += __shfl_xor(cs, 16);
            cs += __shfl_xor(cs, 32);
            const float* mq = a.mu_q + ((size_t)bh * Tm + i) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) dkb[db][r] = fmaf(cs, mq[16 * db + 4 * g + r], dkb[db][r]);
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
                v4i av = reinterpret_cast<const v4i*>(sm.dot)[chunk];
                v4i ak = reinterpret_cast<const v4i*>(sm.qt)[chunk];
                accv = mfma16_i8(av, pop[kq], accv);
                acck = mfma16_i8(ak, dsop[kq], acck);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dvt[db][r] = fmaf((float)accv[r], fv, dvt[db][r]);
                dkt[db][r] = fmaf((float)acck[r], fk, dkt[db][r]);
            }
        }
        __syncthreads();  // dS codes complete in LDS

        // ---- dQ (BQ x D/4 columns of this wave) += dS^ K^
        const float fq = (float)((double)sS * (double)skj * a.scale);
        float* dQ = a.dQ + head + (size_t)qbase * D;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            v4i av = reinterpret_cast<const v4i*>(sm.ds)[g * BQ + 16 * mb + n16];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                v4i acc = mfma16_i8(av, ktop[nb], v4i{0, 0, 0, 0});
                const int dcol = (D / 4) * w + 16 * nb + n16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ql = 16 * mb + 4 * g + r;
                    unsafeAtomicAdd(dQ + (size_t)ql * D + dcol, (float)acc[r] * fq);
                }
            }
        }
        __syncthreads();  // LDS reused by the next tile
    }

    // ---- write dV and dK (lane = key, 4 consecutive d per block)
    float* dV = a.dV + head + (size_t)key * D;
    float* dK = a.dK + head + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        v4f kv;
#pragma unroll
        for (int r = 0; r < 4; ++r) kv[r] = (float)((double)(dkt[db][r] + dkb[db][r]) * a.scale);
        *reinterpret_cast<v4f*>(dV + 16 * db + 4 * g) = dvt[db];
        *reinterpret_cast<v4f*>(dK + 16 * db + 4 * g) = kv;
    }
}

__global__ void zero_f32_kernel(float4* p, size_t n4) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n4; i += stride) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <bool BF16, int D, int BQ>
hipError_t bwd_dispatch(const Dims& d, const BwdArgs& a, hipStream_t s) {
    dim3 grid(d.Tn(), d.BH());
    if (d.causal) {
        if (d.q_smooth) bwd_kernel<BF16, D, BQ, true, true><<<grid, 256, 0, s>>>(a);
        else bwd_kernel<BF16, D, BQ, true, false><<<grid, 256, 0, s>>>(a);
    } else {
        if (d.q_smooth) bwd_kernel<BF16, D, BQ, false, true><<<grid, 256, 0, s>>>(a);
        else bwd_kernel<BF16, D, BQ, false, false><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t bwd_dispatch_bq(const Dims& d, const BwdArgs& a, hipStream_t s) {
    return d.bq == 128 ? bwd_dispatch<BF16, D, 128>(d, a, s) : bwd_dispatch<BF16, D, 64>(d, a, s);
}

}  // namespace

hipError_t launch_bwd(const Dims& d, const sage_qtensors& qk, const sage_dotensors& dos,
                      const float* L, float* dQ, float* dK, float* dV, hipStream_t s) {
    const size_t n4 = (size_t)d.BH() * d.N * d.D / 4;
    zero_f32_kernel<<<(unsigned)std::min<size_t>((n4 + 255) / 256, 4096), 256, 0, s>>>(
        reinterpret_cast<float4*>(dQ), n4);
    BwdArgs a{qk.q,  qk.qt, qk.sq,   qk.k,    qk.kt,     qk.sk,  qk.vr, qk.mu_q, qk.qk_bias, dos.delta,
              dos.dot, dos.sdo, dos.dor, L, dQ, dK, dV, d.N, d.scale};
    if (d.bf16) return d.D == 128 ? bwd_dispatch_bq<true, 128>(d, a, s) : bwd_dispatch_bq<true, 64>(d, a, s);
    return d.D == 128 ? bwd_dispatch_bq<false, 128>(d, a, s) : bwd_dispatch_bq<false, 64>(d, a, s);
}

}  // namespace sage
