// SageBwd INT8 forward (SageBwd method summary, forward steps (3)-(5);
// SageAttention3 write-up Eq. 1 and Eq. 8).
//
// One workgroup = 4 waves = 64 queries of one head; wave w owns 16 queries,
// so a wave holds little state (about 110 registers) and four waves, from
// four independent workgroups, share each SIMD: while some wait on products,
// LDS or their workgroup's barrier, others keep the vector units busy (the
// vector units are the bound: about 190 issue slots per wave and tile against
// 16 products).  Key/value tiles of 64 keys (one K/V quantisation block)
// stream through two LDS stages filled one tile ahead by asynchronous copies:
// the K codes (R32 row tiles) and the V codes (C64P column tiles) are
// contiguous 64*D-byte runs in HBM.
//
// Per tile and wave, on the matrix cores (v_mfma_i32_16x16x64_i8):
//   S^T (64 keys x 16 queries) = K^_j Q^_i^T            int32
// each lane holds the 16 logits of one query (lane % 16) in four key blocks
// of four, the other 48 keys of that query being in the lanes 16, 32 and 48
// away (row statistics: in-lane, then two lane swaps).  Then, in float32 and
// log2 units (x = S * log2 e):
//   rm = rowmax, m = reference maximum (moved lazily, see below),
//   P^ codes = rint(127 * 2^(x - rm))         (= P~ / s_P, independent of m)
//   s_P = 2^(rm - m) / 127,  l += s_P * sum(127 * 2^(x - rm))
// and the codes feed the second product straight from registers:
//   O^T (D x 16 queries) += V^_j^T P^^T  (int32) -> O = O * alpha + f32 * s_P s_V.
// (l and O are kept multiplied by 127, i.e. scaled by 127 s_P = 2^(rm - m):
// no division per tile; the factor cancels in O / l and leaves L as log2 127.)
// The result order of S^T (key 16 kb + 4 g + r in lane group g, register r
// of key block kb) is the operand order of a 64-key contraction once the V
// codes are stored permuted (C64P), so no shuffle or LDS round trip is needed.
#include <climits>
#include <type_traits>

#include "sage_device.h"
#include "sage_internal.h"

namespace sage {
namespace {

struct FwdArgs {
    const int8_t* q;
    const float* sq;
    const int8_t* k;
    const float* sk;
    const int8_t* vt;
    const float* sv;
    const float* qk_bias;
    u16* O;
    float* L;
    int N, bq;
    double scale2;  // softmax scale * log2(e)
};

constexpr int kWaves = 4;
constexpr int kQTile = 16 * kWaves;  // queries per workgroup
constexpr int kKTile = 64;           // keys per stage (= the K/V quantisation block)
constexpr float kLazy = 8.f;         // log2 slack before the reference maximum moves

// Maximum / sum over the four lane groups holding one query (lanes l, l^16,
// l^32, l^48): each lane swap returns a lane's own value and its partner's.
__device__ __forceinline__ float qmax4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ int qmax4i(int x) {
    auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((int)a[0], (int)a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((int)b[0], (int)b[1]);
}
__device__ __forceinline__ float qsum4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
struct FwdStage {
    int8_t k[kKTile * D];          // K codes of the key tile, R32
    int8_t v[kKTile * D];          // V codes of the key tile, C64P
    float bias[kQTile / 64][kKTile];  // Q-smoothing bias rows of the tile's Q blocks
};

// Lowest integer sum a product can hold (|sum| <= 127^2 D < 2^21), as the
// magic-started accumulator sees it: a masked key never wins a row maximum,
// and a row with no visible key in the tile keeps a finite maximum.
constexpr int kMaskedSum = kMagicBits - (1 << 22) + 1;

// F8: the E4M3 variant (codes E4M3, 448 in place of 127, float32 products).
template <bool BF16, int D, bool CAUSAL, bool QSMOOTH, bool PSTATIC, bool F8>
__global__ __launch_bounds__(64 * kWaves, 4) void fwd_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ sq, const int8_t* __restrict__ k,
    const float* __restrict__ sk, const int8_t* __restrict__ vt, const float* __restrict__ sv,
    const float* __restrict__ qk_bias, u16* __restrict__ Out, float* __restrict__ L, int N, int bq,
    double scale2) {
    constexpr int TILE_BYTES = kKTile * D;   // K or V codes of one tile
    constexpr int KS = D / 64;               // contraction steps over d (S^T)
    constexpr int DB = D / 16;               // 16-row blocks of d (O^T)
    constexpr int NT = 64 * kWaves;
    static_assert(TILE_BYTES % 1024 == 0, "stage shape");
    static_assert(!(F8 && PSTATIC), "the static P scale is an INT8 ablation");
    using Acc = typename std::conditional<F8, v4f, v4i>::type;
    constexpr float kLog2Qmax = F8 ? kLog2_448 : kLog2_127;
    __shared__ __align__(16) FwdStage<D> st[2];

    const int Tn = N / kKTile;
    const int Tm = N / bq;
    const int ntiles = (N + kQTile - 1) / kQTile;

    // Workgroup -> (query tile, head).  Blocks are dealt to the eight XCDs
    // round-robin; when the heads divide evenly each XCD owns whole heads
    // (their K/V stay in its L2), and across an XCD's heads the query tiles
    // go heavy first (causal: the last tiles see the most keys).
    int qt, bh;
    {
        const int id = blockIdx.x;
        const int BH = (int)gridDim.x / ntiles;
        int unit;
        if ((BH & 7) == 0) {
            const int xcd = id & 7, k = id >> 3, hpx = BH >> 3;
            bh = xcd + 8 * (k % hpx);
            unit = k / hpx;
        } else {
            bh = id % BH;
            unit = id / BH;
        }
        qt = CAUSAL ? (ntiles - 1 - unit) : unit;
    }
    const size_t head = (size_t)bh * N * D;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, n = lane & 15, g = lane >> 4;
    const int q0 = qt * kQTile + w * 16;
    const bool active = q0 < N;
    const int query = q0 + n;

    int jend = Tn;
    if (CAUSAL) jend = min(Tn, (qt * kQTile + kQTile) / kKTile);

    // Q codes as the B operand of S^T: column = query (lane % 16), 16 bytes
    // of d per lane group and contraction step.
    v4i qop[KS];
    float sqv = 0.f;
    if (active) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qop[ks] = *reinterpret_cast<const v4i*>(q + head + off_r32(query, 64 * ks + 16 * g, D));
        sqv = sq[(size_t)bh * Tm + q0 / bq];
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = v4i{0, 0, 0, 0};
    }

    // the product s_Q * scale * log2 e in float64; each tile multiplies in
    // its s_K and rounds once to float32
    const double sq_s2 = (double)sqv * scale2;
    float m = -INFINITY, l = 0.f;
    v4f o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = v4f{0, 0, 0, 0};
    const v4i magic4 = v4i{kMagicBits, kMagicBits, kMagicBits, kMagicBits};
    const v4f zero4 = v4f{0.f, 0.f, 0.f, 0.f};

    // asynchronous copy of key tile j (K and V codes: two contiguous runs;
    // with Q-smoothing also the tile's 64 bias values of each Q block)
    const unsigned voff = 16u * lane;
    auto load = [&](int j, FwdStage<D>& dst) __attribute__((always_inline)) {
        const int8_t* ks_ = k + head + (size_t)j * TILE_BYTES;
        const int8_t* vs_ = vt + head + (size_t)j * TILE_BYTES;
        const unsigned lk = lds_addr(dst.k), lv = lds_addr(dst.v);
#pragma unroll
        for (int c0 = 0; c0 < TILE_BYTES; c0 += NT * 16) {
            if (c0 + w * 1024 < TILE_BYTES)   // a d=64 tile is half a round
                copy16x2_to_lds(ks_ + c0 + w * 1024, lk + c0 + w * 1024, voff, vs_ + c0 + w * 1024,
                                lv + c0 + w * 1024, voff);
        }
        if (QSMOOTH && w == kWaves - 1) {
            // lane group r of the first max(1, kQTile/bq) groups: Q block row
            // r, 16 B per lane (a row of 64 floats lands in bias[r]); a
            // workgroup narrower than a Q block reads one row
            const int r = lane >> 4;
            const int qb = qt * kQTile / bq + r;
            if (r < max(1, kQTile / bq) && qb < Tm)
                copy16_to_lds(qk_bias + ((size_t)bh * Tm + qb) * N + (size_t)j * kKTile + 4 * (lane & 15),
                              &dst.bias[0][0]);
        }
    };

    if (jend > 0) load(0, st[0]);
    wait_vmem();   // the asynchronous copies are not seen by the compiler's waits
    // the Q codes are complete here, not at their first use inside the loop
    // (after that tile's copies)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qop[ks]);
    __syncthreads();

    for (int j = 0; j < jend; ++j) {
        const FwdStage<D>& cur = st[j & 1];
        if (j + 1 < jend) load(j + 1, st[(j + 1) & 1]);

        const int k0 = j * kKTile;
        const bool wave_on = active && (!CAUSAL || k0 <= q0 + 15);
        if (wave_on) {
            const v4i* lv = reinterpret_cast<const v4i*>(cur.v);
            // S^T for the four 16-key blocks of the tile
            Acc s[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                v4i av[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    av[ks] = *reinterpret_cast<const v4i*>(cur.k + off_r32(16 * kb + n, 64 * ks + 16 * g, D));
                if constexpr (F8) {
                    // d = 128: both chunks in one 16x16x128 product
                    if constexpr (KS == 2) s[kb] = mfma16_f8x128(av[0], av[1], qop[0], qop[1], zero4);
                    else s[kb] = mfma16_f8x64(av[0], qop[0], zero4);
                } else {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) s[kb] = mfma16_i8(av[ks], qop[ks], ks == 0 ? magic4 : s[kb]);
                }
            }
            // one rounding to float32 from the float64 product of the scales
            // (keeps the logits within an ulp of the definition)
            const float c2 = (float)(sq_s2 * (double)sk[(size_t)bh * Tn + j]);
            float rm, sum;
            v4i pc;   // P codes: byte r of dword kb = key 16 kb + 4 g + r
            auto codes = [&](auto mask_tag) __attribute__((always_inline)) {
                constexpr bool MASK = decltype(mask_tag)::value;
                // Row maximum of this tile (log2 units).  Without Q-smoothing the
                // logits are one positive scale times the integer sums, so the
                // maximum is taken on the accumulator bits (which order like the
                // sums); masked keys never win it.
                // with Q-smoothing: the biased logits x = S c2 + bias log2 e,
                // formed once and kept for the codes
                float xq[4][4];
                if (QSMOOTH) {
                    const float* brow = cur.bias[(16 * w) / bq];
                    rm = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const v4f b4 = *reinterpret_cast<const v4f*>(brow + 16 * kb + 4 * g);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = k0 + 16 * kb + 4 * g + r;
                            xq[kb][r] = fmaf(acc_value(s[kb][r]), c2, b4[r] * kLog2e);
                            if (!(MASK && key > query)) rm = fmaxf(rm, xq[kb][r]);
                        }
                    }
                    rm = qmax4(rm);
                } else if constexpr (F8) {
                    // float sums: their maximum, times the positive scale.  Every
                    // row of a wave that reaches here sees key k0 (k0 <= q0).
                    float fm = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = k0 + 16 * kb + 4 * g + r;
                            if (!(MASK && key > query)) fm = fmaxf(fm, s[kb][r]);
                        }
                    rm = qmax4(fm) * c2;
                } else {
                    int im = kMaskedSum;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = k0 + 16 * kb + 4 * g + r;
                            im = max(im, (MASK && key > query) ? kMaskedSum : s[kb][r]);
                        }
                    rm = unmagic(qmax4i(im)) * c2;
                }
                // codes against the tile maximum (per token), or with the
                // static scale against the exact running maximum
                const float shift = (PSTATIC ? fmaxf(m, rm) : rm) - kLog2Qmax;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    uint32_t word = 0u;
                    float ev[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = QSMOOTH ? xq[kb][r] - shift : fmaf(acc_value(s[kb][r]), c2, -shift);
                        if (MASK) {
                            const int key = k0 + 16 * kb + 4 * g + r;
                            if (key > query) x = -INFINITY;
                        }
                        // 127 * 2^(x - rm), in [0, 127] (E4M3: 448 and [0, 448])
                        const float e = __builtin_amdgcn_exp2f(x);
                        sum = (kb == 0 && r == 0) ? e : sum + e;
                        ev[r] = e;
                        // byte r of the word = rint(e) (round to nearest even)
                        if constexpr (!F8) word = __builtin_amdgcn_cvt_pk_u8_f32(e, r, word);
                    }
                    pc[kb] = F8 ? pack_e4m3(ev[0], ev[1], ev[2], ev[3]) : (int)word;
                }
            };
            // Diagonal tiles (some key after some query) take the masked
            // instantiation; every other tile runs without a compare.
            if (CAUSAL && (k0 + kKTile - 1 > q0)) codes(std::true_type{});
            else codes(std::false_type{});
            // Reference maximum: moves only when the row max exceeds it by
            // more than 2^8, so the rescale below is rare.  The codes
            // 127 * 2^(x - rm) do not depend on it, only l and O's common
            // factor do, and those use it consistently.
            // (static scale: the exact running maximum, s_P = 1/127)
            const float m_new = PSTATIC ? fmaxf(m, rm) : ((rm > m + kLazy) ? rm : m);
            // 127 s_P (E4M3: 448 s_P): l and O both carry the factor, which
            // cancels in O / l and is taken out of L at the end
            const float sP = PSTATIC ? 1.f : __builtin_amdgcn_exp2f(rm - m_new);
            if (__builtin_expect(__any(m_new != m), 0)) {
                // rare: a row's reference maximum moved; rescale l and O
                const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first tile
                l *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db] *= alpha;
            }
            // l is kept per lane group (this lane's 16 keys of each tile): sP
            // and alpha are the same for the four groups of a query, so their
            // shares are added once, after the last tile
            l = fmaf(sum, sP, l);
            m = m_new;
            const float beta = sP * sv[(size_t)bh * Tn + j];
            // O^T += V^^T P^^T: one product per 16 rows of d, the 64 keys of the
            // tile as the contraction (V codes C64P, P codes from registers)
            Acc acc[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if constexpr (F8) acc[db] = mfma16_f8x64(lv[g * D + 16 * db + n], pc, zero4);
                else acc[db] = mfma16_i8(lv[g * D + 16 * db + n], pc, magic4);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[db][r] = fmaf(acc_value(acc[db][r]), beta, o[db][r]);
        }
        wait_vmem();       // the next tile has landed
        __syncthreads();   // ... for every wave; this stage may be overwritten
    }

    // O^T block db holds rows d = 16 db + 4 g + r of column (query) n
    if (active) {
        const float lq = qsum4(l);   // the row sum: the four lane groups' shares
        u16* O = Out + head + (size_t)query * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u16 h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = from_f32<BF16>(__fdiv_rn(o[db][r], lq));
            uint2 pk;
            pk.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            pk.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            *reinterpret_cast<uint2*>(O + 16 * db + 4 * g) = pk;
        }
        if (g == 0) L[(size_t)bh * N + query] = (m + (log2f(lq) - kLog2Qmax)) * kLn2;
    }
}

template <bool BF16, int D>
hipError_t fwd_dispatch(const Dims& d, const FwdArgs& a, hipStream_t s) {
    const dim3 grid(((d.N + kQTile - 1) / kQTile) * d.BH());
    const dim3 block(64 * kWaves);
#define SAGE_FWD_ARGS a.q, a.sq, a.k, a.sk, a.vt, a.sv, a.qk_bias, a.O, a.L, a.N, a.bq, a.scale2
#define SAGE_FWD(C, QS)                                                                            \
    (d.fp8        ? fwd_kernel<BF16, D, C, QS, false, true><<<grid, block, 0, s>>>(SAGE_FWD_ARGS)  \
     : d.p_static ? fwd_kernel<BF16, D, C, QS, true, false><<<grid, block, 0, s>>>(SAGE_FWD_ARGS)  \
                  : fwd_kernel<BF16, D, C, QS, false, false><<<grid, block, 0, s>>>(SAGE_FWD_ARGS))
    if (d.causal) {
        if (d.q_smooth) SAGE_FWD(true, true);
        else SAGE_FWD(true, false);
    } else {
        if (d.q_smooth) SAGE_FWD(false, true);
        else SAGE_FWD(false, false);
    }
#undef SAGE_FWD
#undef SAGE_FWD_ARGS
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const Dims& d, const sage_qtensors& qk, void* O, float* L, hipStream_t s) {
    FwdArgs a{qk.q, qk.sq, qk.k, qk.sk, qk.vt, qk.sv, qk.qk_bias, static_cast<u16*>(O), L, d.N, d.bq,
              d.scale * kLog2e_d};
    if (d.bf16) return d.D == 128 ? fwd_dispatch<true, 128>(d, a, s) : fwd_dispatch<true, 64>(d, a, s);
    return d.D == 128 ? fwd_dispatch<false, 128>(d, a, s) : fwd_dispatch<false, 64>(d, a, s);
}

}  // namespace sage
