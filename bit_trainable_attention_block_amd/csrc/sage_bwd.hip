// SageBwd INT8 backward (SageBwd method summary, backward steps (2)-(7);
// SageAttention3 write-up Eq. 9 and its INT8 updates), key blocks outer and
// query blocks inner (paperlayer appendix A.1), in two kernels:
//
// 1. bwd_kernel — one workgroup = 8 waves = two 64-key blocks of one head;
//    wave w owns 16 keys of block 2*jj + w/4 and keeps their dV and dK in
//    float32 registers for the whole sweep over query tiles.  The query tile
//    (BQ rows, the dO/Q quantisation block: Q codes, dO codes in the
//    transposed operand order, dO in 16-bit) streams through a double-buffered
//    LDS stage filled by asynchronous global->LDS copies one tile ahead.  Per
//    tile each wave computes, on the matrix cores (16x16 tiles, lane = key):
//      S  = Q^ K^T     v_mfma_i32_16x16x64_i8            (recompute)
//      dP = dO V^T     v_mfma_f32_16x16x32_{bf16,f16}    (kept in 16-bit)
//    then on the vector units P = 2^(S log2e - L log2e), dS = P (dP - delta);
//    the tile maxima of P and |dS| (one scale per BQ x 64 tile) are reduced
//    in-wave with DPP and across the block's four waves through LDS, and the
//    codes feed, straight from registers,
//      dV^T += dO^^T P^   and   dK^T += Q^^T dS^        (16x16x64 i8)
//    because S's result order is the operand order of the transposed codes
//    (C64P for dO; Q's transposed operand is read from its row tiles with
//    the LDS transpose read).  The dS codes of each tile go to the workspace
//    key-major, two 16-byte stores per lane, and its scale beside them.
// 2. dq_kernel — one workgroup per query tile: dQ_i = sum_j dS^_ij K^_j
//    s_dS,ij s_K,j (INT8 products, float32 across tiles), the dS codes read
//    back transposed by the LDS transpose read.  dQ is written once: no
//    atomics and no clearing pass.
//
// Integer products start from the accumulator 1.5 * 2^23 so that their
// float value is one exact subtraction away (see unmagic).  Codes are
// rounded to nearest-even by one fma with 1.5 * 2^23 and packed with v_perm.
//
// dS workspace layout, per tile (BQ queries x 64 keys, BQ * 64 bytes): key
// row kr (0..63) holds BQ bytes; query q = 16 mb + 4 g + r of the tile sits
// at position p = (BQ/4) g + 4 mb + r, and the 16-byte chunk c of a row is
// stored at chunk slot c ^ (kr mod BQ/16) ^ (bit 4 of kr).  A transpose read
// takes eight consecutive rows in each lane group: the first term spreads
// them over distinct LDS banks, the second gives rows 16 apart (the lane
// groups served together) the other half of the slots.
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "sage_device.h"
#include "sage_internal.h"

namespace sage {
namespace {

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

// x / Q for a tile maximum x >= 0 and the code range Q (127, or 448 for
// E4M3): the product with the rounded reciprocal, then one fma step on the
// exact residual x - q Q.  The quotient is within an ulp of the correctly
// rounded one (it matched it on every one of 3.2 million inputs tried); the P
// and dS scales are compared to tolerance, not bit for bit, and this costs a
// quarter of the instructions of a full division.
template <bool F8>
__device__ __forceinline__ float div_by_qmax(float x) {
    constexpr float Q = F8 ? 448.f : 127.f;
    constexpr float c = 1.f / Q;
    const float q = x * c;
    return fmaf(fmaf(-q, Q, x), c, q);
}

// Byte 0 of four magic-rounded floats -> one dword (rows r = 0..3).
__device__ __forceinline__ int pack_magic(float a, float b, float c, float d) {
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x04000c0cu);
    return (int)(lo | hi);
}

// Workgroup -> (unit, head); `units` is the number of units per head.
// Blocks are dealt to the eight XCDs round-robin; when the heads divide
// evenly each XCD owns whole heads.  UNITS_OUTER = false: the XCD works
// through its heads one after another, units in order (a head's streamed
// tiles stay in that XCD's L2).  UNITS_OUTER = true: unit-major across the
// XCD's heads (the first units, the heaviest, start first).
template <bool UNITS_OUTER>
__device__ __forceinline__ void xcd_coords(int units, int BH, int& unit, int& bh) {
    const int id = blockIdx.x;
    if ((BH & 7) == 0) {
        const int xcd = id & 7, k = id >> 3, hpx = BH >> 3;
        if (UNITS_OUTER) { unit = k / hpx; bh = xcd + 8 * (k % hpx); }
        else { bh = xcd + 8 * (k / units); unit = k % units; }
    } else {
        bh = id / units;
        unit = id % units;
    }
}

// Q codes in a backward stage: the R32 16-byte chunk at byte offset `off` is
// stored at qswz(off), which flips chunk bit 3 where chunk bit 4 is set (bit
// 4 of a chunk index is bit 4 of its row).  The transposed reads of the dK
// product take rows r and r + 16 of a chunk column in lane groups that the
// LDS serves together; unswizzled both rows land on the same banks.  The
// row-major reads of the S product stay on 16 consecutive chunks.
__device__ __forceinline__ int qswz(int off) { return off ^ (((off >> 8) & 1) << 7); }

template <int BQ, int D, bool DPI8>
struct BwdStage {
    int8_t q[BQ * D];     // Q codes, R32
    int8_t dot[BQ * D];   // dO codes, C64P
    int8_t dor[(DPI8 ? 1 : 2) * BQ * D];   // dO, 16-bit row tiles (R16H order); with dp_int8 dO's codes, R32
    float l2[BQ];         // L * log2 e
    float ndelta[BQ];     // -delta (the dP accumulation starts from it)
};

// The 16-bit dO sits in the stage in 16-row tiles: element (row, col) of a
// 16-row group at ((col / 8) * 16 + row % 16) * 8 + col % 8, so that the dP
// product's A operand (a row's 8 consecutive d per lane) is one 16-byte read
// per lane with the 16 rows of a lane group on distinct banks.  The stage is
// filled from the row-major dO: the wave's copy of stage bytes [off, off +
// 1 KiB) reads, for lane l, the 16 bytes of row 16 grp + l % 16 at chunk
// column rem0 / 16 + l / 16 (grp, rem0: the 16-row group and the chunk
// offset in it of the copy's first chunk); the lane part is voff_dor.
template <int D>
__device__ __forceinline__ int r16h_src_off(int off) {
    constexpr int G16 = 2 * D;   // 16-byte chunks per 16-row group
    const int c0 = off >> 4;     // the copy's first chunk (a multiple of 64)
    return (c0 / G16) * 16 * 2 * D + ((c0 % G16) >> 4) * 16;
}

// Asynchronous copy of query tile qbase (Q codes, dO codes, dO) into the
// stage at LDS address `lds`; the Q codes land swizzled (qswz), which the
// copy does by reading lane l's chunk from qswz(16 l) (voff_q), and the
// 16-bit dO lands in its row-tile order (r16h_src_off, voff_dor).  The three
// regions are BQ*D, BQ*D and 2*BQ*D bytes (BQ*D for the third with dp_int8:
// dO's R32 codes, copied as they are), laid out in the same order in the
// stage; each wave instruction moves 1 KiB, and round u of the eight waves
// moves the stage's u-th 8 KiB.  When a region is a whole number of rounds
// (BQ*D a multiple of 8 KiB) the region of a round is known at compile time.
// voff = 16 * lane.
template <int BQ, int D, bool DPI8>
struct StagePlan {
    static constexpr int QB = BQ * D, TOT = (DPI8 ? 3 : 4) * QB, R = 8 * 1024;
    static constexpr int ROUNDS = (TOT + R - 1) / R, FULL = TOT / R;
    static_assert(QB % 1024 == 0, "stage shape");
    const int8_t* src[ROUNDS];
    unsigned dst[ROUNDS], vo[ROUNDS];
};

template <int BQ, int D, bool DPI8>
__device__ __forceinline__ void plan_query_tile(StagePlan<BQ, D, DPI8>& pl, unsigned lds, const int8_t* q,
                                                const int8_t* dot, const int8_t* dorb, int w, unsigned voff,
                                                unsigned voff_q, unsigned voff_dor) {
    using P = StagePlan<BQ, D, DPI8>;
    constexpr int QB = P::QB, R = P::R, ROUNDS = P::ROUNDS;
    const int8_t** src = pl.src;
    unsigned* dst = pl.dst;
    unsigned* vo = pl.vo;
    // source of the dO region's bytes [off, off + 1 KiB)
    auto dor_src = [&](int off) __attribute__((always_inline)) {
        return DPI8 ? dorb + off : dorb + r16h_src_off<D>(off);
    };
    const unsigned vo_dor = DPI8 ? voff : voff_dor;
#pragma unroll
    for (int u = 0; u < ROUNDS; ++u) {
        const int c0 = u * R + w * 1024;
        if constexpr (QB % R == 0) {
            constexpr int RQ = QB / R;   // rounds per 1-byte region
            const int off = (u % RQ) * R + w * 1024;
            src[u] = u < RQ ? q + off : u < 2 * RQ ? dot + off : dor_src((u - 2 * RQ) * R + w * 1024);
            vo[u] = u < RQ ? voff_q : u < 2 * RQ ? voff : vo_dor;
        } else {
            src[u] = c0 < QB ? q + c0 : c0 < 2 * QB ? dot + (c0 - QB) : dor_src(c0 - 2 * QB);
            vo[u] = c0 < QB ? voff_q : c0 < 2 * QB ? voff : vo_dor;
        }
        dst[u] = lds + c0;
    }
}

// Round u of a planned stage copy (one instruction per wave).  The plan's
// source and LDS addresses are wave-uniform; where the compiler has kept one
// in a vector register across the products, readfirstlane brings it back to a
// scalar register for the copy (a no-op for one already there).
__device__ __forceinline__ const int8_t* uniform_ptr(const int8_t* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<const int8_t*>(((uint64_t)hi << 32) | lo);
}
template <int BQ, int D, bool DPI8>
__device__ __forceinline__ void issue_round(const StagePlan<BQ, D, DPI8>& pl, int u, int w) {
    using P = StagePlan<BQ, D, DPI8>;
    // the last round of a stage that is not a whole number of rounds covers
    // only some waves
    if (u < P::FULL || P::FULL * P::R + w * 1024 < P::TOT)
        copy16x1_to_lds(uniform_ptr(pl.src[u]), __builtin_amdgcn_readfirstlane(pl.dst[u]), pl.vo[u]);
}

// The whole stage at once.
template <int BQ, int D, bool DPI8>
__device__ __forceinline__ void stage_query_tile(unsigned lds, const int8_t* q, const int8_t* dot,
                                                 const int8_t* dorb, int w, unsigned voff, unsigned voff_q,
                                                 unsigned voff_dor) {
    using P = StagePlan<BQ, D, DPI8>;
    StagePlan<BQ, D, DPI8> pl;
    plan_query_tile<BQ, D, DPI8>(pl, lds, q, dot, dorb, w, voff, voff_q, voff_dor);
    copy16_rounds<P::FULL>(pl.src, pl.dst, pl.vo);
    if constexpr (P::FULL < P::ROUNDS) issue_round<BQ, D, DPI8>(pl, P::FULL, w);
}

// Two LDS stages alternate: tile i is read from stage (i - istart) & 1 while
// the next tile is copied into the other one.
// F8: the E4M3 variant (codes E4M3, 448 in place of 127, float32 products).
template <bool BF16, int D, int BQ, bool CAUSAL, bool QSMOOTH, bool DPI8, bool F8>
__global__ __launch_bounds__(512, 1) void bwd_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ sq, const int8_t* __restrict__ k,
    const float* __restrict__ sk, const u16* __restrict__ V, const int8_t* __restrict__ vr8,
    const float* __restrict__ sv, const float* __restrict__ mu_q,
    const float* __restrict__ qk_bias, const float* __restrict__ delta, const int8_t* __restrict__ dot,
    const float* __restrict__ sdo, const u16* __restrict__ dO16, const int8_t* __restrict__ dor8,
    const float* __restrict__ L,
    int8_t* __restrict__ dsw, float* __restrict__ sds, float* __restrict__ dK, float* __restrict__ dV, int N,
    int BH, double scale) {
    constexpr int MB = BQ / 16;   // 16-query blocks per tile
    constexpr int KQ = BQ / 64;   // i8 contraction steps over queries
    constexpr int KS8 = D / 64;   // i8 contraction steps over d
    constexpr int KSH = D / 32;   // 16-bit contraction steps over d
    constexpr int DB = D / 16;    // 16-wide blocks of d
    constexpr int CH = BQ / 16;   // 16-byte chunks per dS key row
    static_assert(!(F8 && DPI8), "the INT8 dP ablation has no E4M3 form");
    using Acc = typename std::conditional<F8, v4f, v4i>::type;
    constexpr float kQmax = F8 ? 448.f : 127.f;
    __shared__ __align__(16) BwdStage<BQ, D, DPI8> st[2];
    using Stage = BwdStage<BQ, D, DPI8>;
    static_assert(offsetof(Stage, dot) == BQ * D && offsetof(Stage, dor) == 2 * BQ * D, "stage layout");
    __shared__ float red[2][2][4];   // [key block][P | dS][key group]

    const int Tn = N / 64, Tm = N / BQ;
    int jj, bh;
    xcd_coords<false>((Tn + 1) / 2, BH, jj, bh);
    const size_t head = (size_t)bh * N * D;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63, n16 = lane & 15, g = lane >> 4;
    const unsigned voff = 16u * lane, voff_q = (unsigned)qswz(16 * lane);
    const unsigned voff_dor = (unsigned)((lane & 15) * 2 * D + (lane >> 4) * 16);
    // this lane's Q chunk offsets in a stage (swizzled): the S product reads
    // row 16 mb + n16, chunk column 4 ks + g, at qa_lane[mb & 1] + (mb / 2)
    // 32 D + 2048 ks; the dK product's transposed reads take query row
    // 64 kq + 16 (kk / 4) + 4 g + kk % 4 (+ 32), bytes 8 hf.., of chunk column
    // db at tr_lane + 64 D kq (+ 32 D) + 512 db (kk = n16 / 2, hf = n16 % 2)
    const int qa_lane[2] = {qswz(off_r32(n16, 16 * g, D)), qswz(off_r32(16 + n16, 16 * g, D))};
    const int tr_lane = qswz((16 * ((n16 >> 1) >> 2) + 4 * g + ((n16 >> 1) & 3)) << 4) + 8 * (n16 & 1);
    const int kb = w >> 2, kg = w & 3;
    const int j = 2 * jj + kb;        // this wave's key block
    const bool kv_on = j < Tn;        // the second block of a ragged tail may not exist
    const int kr = 16 * kg + n16;     // key row inside the block
    const int key = j * 64 + kr;

    // A key block past a ragged end computes on zero operands and stores
    // nothing; keeping it in the same straight-line code as the others
    // avoids merging two paths over the accumulators on every tile.
    // V as the B operand of dP: 16-bit row tiles, or with dp_int8 its codes
    constexpr int KSV = DPI8 ? KS8 : KSH;
    v4i kop[KS8], vop[KSV];
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) kop[ks] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) vop[ks] = v4i{0, 0, 0, 0};
    float skj = 0.f, svj = 0.f;
    if (kv_on) {
#pragma unroll
        for (int ks = 0; ks < KS8; ++ks)
            kop[ks] = *reinterpret_cast<const v4i*>(k + head + off_r32(key, 64 * ks + 16 * g, D));
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
            vop[ks] = DPI8 ? *reinterpret_cast<const v4i*>(vr8 + head + off_r32(key, 64 * ks + 16 * g, D))
                           : *reinterpret_cast<const v4i*>(V + head + (size_t)key * D + 32 * ks + 8 * g);
        skj = sk[(size_t)bh * Tn + j];
        if (DPI8) svj = sv[(size_t)bh * Tn + j];
    }

    v4f dvt[DB], dkt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dvt[db] = v4f{0, 0, 0, 0};
        dkt[db] = v4f{0, 0, 0, 0};
    }
    const v4i magic4 = v4i{kMagicBits, kMagicBits, kMagicBits, kMagicBits};
    const v4f zero4 = v4f{0.f, 0.f, 0.f, 0.f};

    const double skj_s2 = (double)skj * scale * kLog2e_d;   // s_K * scale * log2 e
    const size_t tph = tiles_per_head<BQ, CAUSAL>(Tm, Tn);
    const int istart = CAUSAL ? (2 * jj * 64) / BQ : 0;
    const float* Lh = L + (size_t)bh * N;
    const float* dlh = delta + (size_t)bh * N;
    const int8_t* qh = q + head;
    const int8_t* doth = dot + head;
    constexpr int DOR_B = DPI8 ? 1 : 2;   // bytes per element of the dP operand copy of dO
    const int8_t* dorh = DPI8 ? dor8 + head : reinterpret_cast<const int8_t*>(dO16 + head);
    // Q-smoothing bias of this lane's key for the current query tile, loaded
    // one tile ahead (a key past a ragged end reads nothing)
    float nbias = 0.f;
    if (QSMOOTH && kv_on) nbias = qk_bias[((size_t)bh * Tm + istart) * N + key];

    // dS codes and scale of the last tile, not yet stored
    v4i pend_ds[KQ];
    size_t pend_t = 0;
    float pend_s = 0.f;
    bool pend_on = false;

    // One query tile, read from `cur`; the next one is copied into `nxt`.
    auto step = [&](int i, BwdStage<BQ, D, DPI8>& cur, BwdStage<BQ, D, DPI8>& nxt) __attribute__((always_inline)) {
        const int qbase = i * BQ;
        const bool more = i + 1 < Tm;
        const float biasv = nbias;
        // small loads of the next tile first: waiting for them never waits
        // for the copies issued after them
        float nL = 0.f, nd = 0.f;
        if (more && tid < BQ) {
            nL = Lh[qbase + BQ + tid];
            nd = dlh[qbase + BQ + tid];
        }
        if (QSMOOTH && kv_on && more) nbias = qk_bias[((size_t)bh * Tm + i + 1) * N + key];
        // the previous tile's dS codes and scale go out now, ahead of this
        // tile's copies, so that the wait for the copies at the end of this
        // tile does not also wait for the stores to complete
        if (pend_on) {
            int8_t* drow = dsw + pend_t * (BQ * 64) + kr * BQ;
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                const int slot = (KQ * g + kq) ^ (kr & (CH - 1)) ^ ((kr >> 4) & 1);
                *reinterpret_cast<v4i*>(drow + slot * 16) = pend_ds[kq];
            }
            if (kg == 0 && lane == 0) sds[pend_t] = pend_s;
        }
        // the next tile's copies: one round per 16-query block of the S and
        // dP products below, so that no wave stalls on the load path at once.
        // On the last tile the current tile is copied again into the idle
        // stage (every wave finished reading it before the barrier that ended
        // the previous tile): the copies stay unconditional, and no branch
        // splits the product loop (a branch there lets the compiler sink all
        // the vector work below all the products).
        using Plan = StagePlan<BQ, D, DPI8>;
        Plan pl;
        const int qnext = more ? qbase + BQ : qbase;
        plan_query_tile<BQ, D, DPI8>(pl, lds_addr(&nxt), qh + (size_t)qnext * D, doth + (size_t)qnext * D,
                                     dorh + (size_t)DOR_B * qnext * D, w, voff, voff_q, voff_dor);
        auto issue_rounds_of_block = [&](int mb) __attribute__((always_inline)) {
#pragma unroll
            for (int u = mb * Plan::ROUNDS / MB; u < (mb + 1) * Plan::ROUNDS / MB; ++u) issue_round<BQ, D, DPI8>(pl, u, w);
        };

        // the tile exists and has a visible key (it is stored for the dQ pass)
        const bool tile_on = kv_on && (!CAUSAL || j * 64 <= qbase + BQ - 1);
        const float sqi = sq[(size_t)bh * Tm + i];
        const float sdoi = sdo[(size_t)bh * Tm + i];
        // Tile maxima over the key block's four waves, then the scales.  Raw
        // barrier: the copy of the next tile stays in flight.
        auto tile_scales = [&](float pmax, float dsmax, float& sP, float& sS) __attribute__((always_inline)) {
            pmax = wave_max_nonneg(pmax);
            dsmax = wave_max_nonneg(dsmax);
            if (lane == 0) {
                red[kb][0][kg] = pmax;
                red[kb][1][kg] = dsmax;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            pmax = fmaxf(fmaxf(red[kb][0][0], red[kb][0][1]), fmaxf(red[kb][0][2], red[kb][0][3]));
            dsmax = fmaxf(fmaxf(red[kb][1][0], red[kb][1][1]), fmaxf(red[kb][1][2], red[kb][1][3]));
            sP = div_by_qmax<F8>(pmax);
            sS = div_by_qmax<F8>(dsmax);
        };
        {
            float p[MB][4], ds[MB][4];
            float pmax = 0.f, dsmax = 0.f;
            const float c2 = (float)((double)sqi * skj_s2);  // one rounding from float64
            float bias2 = 0.f;
            if (QSMOOTH) bias2 = (float)((double)biasv * kLog2e_d);
            // ---- S and dP for this wave's 16 keys and all BQ queries, one
            // 16-query block ahead of the vector work on the previous block
            Acc s[MB];
            // dP in float32 from 16-bit operands, or with dp_int8 as an INT8
            // product with dP = f32(sum) * f32(s_dO * s_V) (one rounding)
            using DpT = typename std::conditional<DPI8, v4i, v4f>::type;
            DpT dp[MB];
            const float cdp = DPI8 ? (float)((double)sdoi * (double)svj) : 0.f;
            // LDS operands of a 16-query block are read one block before its
            // products are issued, so the products never wait on LDS
            struct OpsA {
                v4i q[KS8];
                v4i d[KSV];
                v4f nd;   // -delta of the block's four query rows of this lane group
            };
            OpsA opa[2];
            v4f ndb[2];   // dp_int8: -delta of the block issued last and of the one before
            auto read_block = [&](int mb, OpsA& o) __attribute__((always_inline)) {
                const int row = 16 * mb + n16;  // query row (in tile) this lane supplies
#pragma unroll
                for (int ks = 0; ks < KS8; ++ks)
                    o.q[ks] = *reinterpret_cast<const v4i*>(cur.q + qa_lane[mb & 1] + (mb >> 1) * 32 * D + ks * 2048);
#pragma unroll
                for (int ks = 0; ks < KSV; ++ks)
                    o.d[ks] = DPI8 ? *reinterpret_cast<const v4i*>(cur.dor + off_r32(row, 64 * ks + 16 * g, D))
                                   : *reinterpret_cast<const v4i*>(cur.dor + 2 * off_r16h(row, 32 * ks + 8 * g, D));
                o.nd = *reinterpret_cast<const v4f*>(&cur.ndelta[16 * mb + 4 * g]);
            };
            auto mfma_block = [&](int mb, const OpsA& o) __attribute__((always_inline)) {
                if constexpr (F8) {
                    if constexpr (KS8 == 2) s[mb] = mfma16_f8x128(o.q[0], o.q[1], kop[0], kop[1], zero4);
                    else s[mb] = mfma16_f8x64(o.q[0], kop[0], zero4);
                } else {
#pragma unroll
                    for (int ks = 0; ks < KS8; ++ks) s[mb] = mfma16_i8(o.q[ks], kop[ks], ks == 0 ? magic4 : s[mb]);
                }
#pragma unroll
                for (int ks = 0; ks < KSV; ++ks) {
                    // 16-bit dP accumulates onto -delta: the product yields dP - delta
                    if constexpr (DPI8) dp[mb] = mfma16_i8(o.d[ks], vop[ks], ks == 0 ? magic4 : dp[mb]);
                    else dp[mb] = mfma16_h<BF16>(o.d[ks], vop[ks], ks == 0 ? o.nd : dp[mb]);
                }
                if constexpr (DPI8) ndb[mb & 1] = o.nd;
            };
            read_block(0, opa[0]);
            if (MB > 1) read_block(1, opa[1]);
            mfma_block(0, opa[0]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const v4f l2 = *reinterpret_cast<const v4f*>(&cur.l2[16 * mb + 4 * g]);
                if (mb + 2 < MB) read_block(mb + 2, opa[mb & 1]);
                if (mb + 1 < MB) mfma_block(mb + 1, opa[(mb + 1) & 1]);
                issue_rounds_of_block(mb);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = fmaf(acc_value(s[mb][r]), c2, -l2[r]);
                    if (QSMOOTH) x += bias2;
                    const float pv = __builtin_amdgcn_exp2f(x);
                    // dP - delta (16-bit dP already holds it; the INT8 one is scaled here)
                    float dpd;
                    if constexpr (DPI8) dpd = fmaf(unmagic(dp[mb][r]), cdp, ndb[mb & 1][r]);
                    else dpd = dp[mb][r];
                    const float dsv = pv * dpd;
                    p[mb][r] = pv;
                    ds[mb][r] = dsv;
                    pmax = fmaxf(pmax, pv);
                    dsmax = fmaxf(dsmax, fabsf(dsv));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (CAUSAL && (j * 64 + 63 > qbase)) {
                // diagonal (or invisible) tile: zero the keys after each query
                // (by selection, so an overflowed exp there never reaches a
                // product) and take the maxima again
                pmax = 0.f;
                dsmax = 0.f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool vis = key <= qbase + 16 * mb + 4 * g + r;
                        p[mb][r] = vis ? p[mb][r] : 0.f;
                        ds[mb][r] = vis ? ds[mb][r] : 0.f;
                        pmax = fmaxf(pmax, p[mb][r]);
                        dsmax = fmaxf(dsmax, fabsf(ds[mb][r]));
                    }
            }
            float sP, sS;
            tile_scales(pmax, dsmax, sP, sS);
            // hardware reciprocal (within an ulp): a code moves only where
            // P / s_P lies within about 1e-5 of a rounding boundary
            struct OpsB {
                v4i av[KQ];
                v4i ak[KQ];
            };
            OpsB opb[2];
            auto read_db = [&](int db, OpsB& o) __attribute__((always_inline)) {
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) {
                    o.av[kq] = reinterpret_cast<const v4i*>(cur.dot)[kq * 4 * D + g * D + 16 * db + n16];
                    const v2i r1 = lds_read_tr8(cur.q + tr_lane + kq * 64 * D + db * 512);
                    const v2i r2 = lds_read_tr8(cur.q + tr_lane + kq * 64 * D + 32 * D + db * 512);
                    o.ak[kq] = v4i{r1[0], r1[1], r2[0], r2[1]};
                }
            };
            read_db(0, opb[0]);
            if (DB > 1) read_db(1, opb[1]);
            __builtin_amdgcn_sched_barrier(0);
            const float invP = sP > 0.f ? __builtin_amdgcn_rcpf(sP) : 0.f;
            const float invS = sS > 0.f ? __builtin_amdgcn_rcpf(sS) : 0.f;
            // ---- codes, query-contiguous per lane (4 queries per dword)
            v4i pop[KQ], dsop[KQ];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float pc[4], sc[4];
                if constexpr (F8) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pc[r] = p[mb][r] * invP;
                        sc[r] = ds[mb][r] * invS;
                    }
                    pop[mb >> 2][mb & 3] = pack_e4m3(pc[0], pc[1], pc[2], pc[3]);
                    dsop[mb >> 2][mb & 3] = pack_e4m3(sc[0], sc[1], sc[2], sc[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pc[r] = fmaf(p[mb][r], invP, kMagic);  // rint(P / s_P) in the low byte
                        sc[r] = fmaf(ds[mb][r], invS, kMagic);
                    }
                    pop[mb >> 2][mb & 3] = pack_magic(pc[0], pc[1], pc[2], pc[3]);
                    dsop[mb >> 2][mb & 3] = pack_magic(sc[0], sc[1], sc[2], sc[3]);
                }
            }
            // ---- dS codes and scale for the workspace (key-major, swizzled),
            // stored at the start of the next tile
            pend_t = (size_t)bh * tph + tile_index<BQ, CAUSAL>(i, j, Tn);
            pend_on = tile_on;
            pend_s = sS;
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) pend_ds[kq] = dsop[kq];
            if (QSMOOTH) {
                // dK bias (dS^T 1) mu_Q^T from the unquantised dS
                float cs = 0.f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) cs += ds[mb][r];
                cs += __shfl_xor(cs, 16);
                cs += __shfl_xor(cs, 32);
                const float* mq = mu_q + ((size_t)bh * Tm + i) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const v4f m4 = *reinterpret_cast<const v4f*>(mq + 16 * db + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dkt[db][r] = fmaf(cs, m4[r], dkt[db][r]);
                }
            }
            // ---- dV^T += dO^^T P^,  dK^T += Q^^T dS^
            const float fv = sP * sdoi;
            const float fk = sS * sqi;
            Acc accv[DB], acck[DB];
            auto mfma_db = [&](int db, const OpsB& o) __attribute__((always_inline)) {
                const v4i* av = o.av;
                const v4i* ak = o.ak;
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) {
                    if constexpr (!F8) {
                        accv[db] = mfma16_i8(av[kq], pop[kq], kq == 0 ? magic4 : accv[db]);
                        acck[db] = mfma16_i8(ak[kq], dsop[kq], kq == 0 ? magic4 : acck[db]);
                    }
                }
                if constexpr (F8) {
                    // both 64-query chunks in one 16x16x128 product (bq = 128)
                    if constexpr (KQ == 2) {
                        accv[db] = mfma16_f8x128(av[0], av[1], pop[0], pop[1], zero4);
                        acck[db] = mfma16_f8x128(ak[0], ak[1], dsop[0], dsop[1], zero4);
                    } else {
                        accv[db] = mfma16_f8x64(av[0], pop[0], zero4);
                        acck[db] = mfma16_f8x64(ak[0], dsop[0], zero4);
                    }
                }
            };
            // one d-block of products ahead of the accumulation of the previous
            mfma_db(0, opb[0]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if (db + 2 < DB) read_db(db + 2, opb[db & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (db + 1 < DB) mfma_db(db + 1, opb[(db + 1) & 1]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dvt[db][r] = fmaf(acc_value(accv[db][r]), fv, dvt[db][r]);
                    dkt[db][r] = fmaf(acc_value(acck[db][r]), fk, dkt[db][r]);
                }
                settle(dvt[db]);
                settle(dkt[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (more && tid < BQ) {
            asm volatile("" : "+v"(nL), "+v"(nd));   // keep the conversion here, after the work
            nxt.l2[tid] = (float)((double)nL * kLog2e_d);
            nxt.ndelta[tid] = -nd;
        }
        wait_vmem();       // the asynchronous copies are not seen by the compiler's waits
        if (QSMOOTH) settle(nbias);
        __syncthreads();   // the next tile has landed in LDS for every wave; `cur` may be overwritten
    };

    // ---- prologue: first query tile into st0
    stage_query_tile<BQ, D, DPI8>(lds_addr(&st[0]), qh + (size_t)istart * BQ * D, doth + (size_t)istart * BQ * D,
                                  dorh + (size_t)DOR_B * istart * BQ * D, w, voff, voff_q, voff_dor);
    if (tid < BQ) {
        st[0].l2[tid] = (float)((double)Lh[istart * BQ + tid] * kLog2e_d);
        st[0].ndelta[tid] = -dlh[istart * BQ + tid];
    }
    wait_vmem();       // the asynchronous copies are not seen by the compiler's waits
    // the operands held in registers are complete here, not at their first
    // use inside the loop (after that tile's copies)
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) settle(kop[ks]);
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) settle(vop[ks]);
    if (QSMOOTH) settle(nbias);
    __syncthreads();
    for (int i = istart; i < Tm; ++i) {
        const int b = (i - istart) & 1;
        step(i, st[b], st[b ^ 1]);
    }
    if (pend_on) {
        int8_t* drow = dsw + pend_t * (BQ * 64) + kr * BQ;
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
            const int slot = (KQ * g + kq) ^ (kr & (CH - 1)) ^ ((kr >> 4) & 1);
            *reinterpret_cast<v4i*>(drow + slot * 16) = pend_ds[kq];
        }
        if (kg == 0 && lane == 0) sds[pend_t] = pend_s;
    }

    // ---- write dV and dK (lane = key, 4 consecutive d per block)
    if (kv_on) {
        float* dVk = dV + head + (size_t)key * D;
        float* dKk = dK + head + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            v4f kv;
#pragma unroll
            for (int r = 0; r < 4; ++r) kv[r] = (float)((double)dkt[db][r] * scale);
            *reinterpret_cast<v4f*>(dVk + 16 * db + 4 * g) = dvt[db];
            *reinterpret_cast<v4f*>(dKk + 16 * db + 4 * g) = kv;
        }
    }
}

// dQ_i = scale * sum_j s_dS,ij s_K,j M(dS^_ij, K^_j), one workgroup per query
// tile; wave w owns the BQ/4 dS positions [w BQ/4, (w+1) BQ/4) (queries
// 16 mb + 4 w + r) and all D columns.  Each key tile (its dS codes and the
// K codes) streams through a ring of three LDS stages filled two tiles ahead
// by asynchronous copies; the dS codes, read once, are copied with the
// non-temporal hint so that they do not push the K codes (read again by every
// query tile of the head) out of L2.  K's codes arrive as R32 row tiles (swizzled as the
// backward's Q codes are) and are read transposed: column d of a product's B
// operand is two transpose reads of eight keys.
template <int BQ, int D>
struct DqStage {
    int8_t ds[BQ * 64];   // dS codes of one tile, key-major (workspace layout)
    int8_t k[64 * D];     // K codes of the key block, R32, qswz-swizzled
};

template <int D, int BQ, bool CAUSAL, bool F8>
__global__ __launch_bounds__(256, 2) void dq_kernel(const int8_t* __restrict__ dsw, const float* __restrict__ sds,
                                                   const int8_t* __restrict__ k, const float* __restrict__ sk,
                                                   float* __restrict__ dQ, int N, int BH, double scale) {
    constexpr int QPW = BQ / 4;           // positions per wave
    constexpr int MBq = QPW / 16;
    constexpr int NB = D / 16;
    constexpr int CH = BQ / 16;
    constexpr int DS_BYTES = BQ * 64;
    constexpr int K_BYTES = 64 * D;
    constexpr int ROUNDS = (DS_BYTES + K_BYTES) / 4096;
    static_assert((DS_BYTES + K_BYTES) % 4096 == 0 && DS_BYTES % 1024 == 0, "stage shape");
    __shared__ __align__(16) DqStage<BQ, D> st[3];
    using Stage = DqStage<BQ, D>;
    static_assert(offsetof(Stage, k) == DS_BYTES, "stage layout");

    const int Tn = N / 64, Tm = N / BQ;
    int unit, bh;
    xcd_coords<true>(Tm, BH, unit, bh);
    const int i = CAUSAL ? (Tm - 1 - unit) : unit;  // heavy tiles first
    const size_t head = (size_t)bh * N * D;
    const size_t tph = tiles_per_head<BQ, CAUSAL>(Tm, Tn);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, n16 = lane & 15, g = lane >> 4;
    const int jend = CAUSAL ? (i + 1) * BQ / 64 : Tn;

    const unsigned voff = 16u * lane, voff_q = (unsigned)qswz(16 * lane);
    // this lane's K transpose-read offsets (keys 16 g + 8 h + n16 / 2, bytes
    // 8 (n16 % 2).. of chunk column 0); chunk column nb adds 512 nb, which
    // the swizzle (bits 7 and 8) does not see
    int tk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) tk[h] = qswz(off_r32(16 * g + 8 * h + (n16 >> 1), 0, D)) + 8 * (n16 & 1);
    // the stage's ds and k regions are contiguous: round u fills its bytes
    // [4096 u, 4096 u + 4096)
    auto load = [&](int j, DqStage<BQ, D>& st) __attribute__((always_inline)) {
        const size_t t = (size_t)bh * tph + tile_index<BQ, CAUSAL>(i, j, Tn);
        const int8_t* s1 = dsw + t * DS_BYTES;
        const int8_t* s2 = k + head + (size_t)j * K_BYTES;
        const unsigned base = lds_addr(&st);
        const int8_t* src[ROUNDS];
        unsigned dst[ROUNDS], vo[ROUNDS];
#pragma unroll
        for (int u = 0; u < ROUNDS; ++u) {
            const int c0 = u * 4096 + w * 1024;
            const bool is_ds = DS_BYTES % 4096 == 0 ? u * 4096 < DS_BYTES : c0 < DS_BYTES;
            src[u] = is_ds ? s1 + c0 : s2 + (c0 - DS_BYTES);
            dst[u] = base + c0;
            vo[u] = is_ds ? voff : voff_q;
        }
#pragma unroll
        for (int u = 0; u < ROUNDS; ++u) {
            if (u * 4096 + 4096 <= DS_BYTES) copy16x1_nt_to_lds(src[u], dst[u], vo[u]);
            else copy16x1_to_lds(src[u], dst[u], vo[u]);
        }
    };

    v4f acc[MBq][NB];
#pragma unroll
    for (int mb = 0; mb < MBq; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = v4f{0, 0, 0, 0};
    const v4i magic4 = v4i{kMagicBits, kMagicBits, kMagicBits, kMagicBits};

    auto step = [&](int j, DqStage<BQ, D>& cur, DqStage<BQ, D>& nxt) __attribute__((always_inline)) {
        const size_t t = (size_t)bh * tph + tile_index<BQ, CAUSAL>(i, j, Tn);
        const float cj = (float)((double)sds[t] * (double)sk[(size_t)bh * Tn + j] * scale);
        if (j + 2 < jend) load(j + 2, nxt);
        // A = dS^ rows (positions), k = keys 16 g + e, read transposed from the
        // key-major rows: two transpose reads of eight keys each
        v4i av[MBq];
#pragma unroll
        for (int mb = 0; mb < MBq; ++mb) {
            const int c = (QPW * w + 16 * mb) >> 4;
            v2i r[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int krow = 16 * g + 8 * h + (n16 >> 1);
                const int slot = c ^ (krow & (CH - 1)) ^ ((krow >> 4) & 1);
                r[h] = lds_read_tr8(cur.ds + krow * BQ + slot * 16 + 8 * (n16 & 1));
            }
            av[mb] = v4i{r[0][0], r[0][1], r[1][0], r[1][1]};
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            // K^ column d = 16 nb + n16, k = key 16 g + e
            const v2i b0 = lds_read_tr8(cur.k + tk[0] + 512 * nb);
            const v2i b1 = lds_read_tr8(cur.k + tk[1] + 512 * nb);
            const v4i bv = v4i{b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
            for (int mb = 0; mb < MBq; ++mb) {
                if constexpr (F8) {
                    const v4f x = mfma16_f8x64(av[mb], bv, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mb][nb][r] = fmaf(x[r], cj, acc[mb][nb][r]);
                } else {
                    const v4i x = mfma16_i8(av[mb], bv, magic4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mb][nb][r] = fmaf(unmagic(x[r]), cj, acc[mb][nb][r]);
                }
            }
        }
        // tile j + 1 has landed once only tile j + 2's copies (ROUNDS per
        // wave, the only vector memory operations of the loop) may be in
        // flight; the compiler's own waits do not see these copies
        if (j + 2 < jend) wait_vmem_leave<ROUNDS>();
        else wait_vmem();
        __syncthreads();   // tile j + 1 landed for every wave; stage j may be overwritten
    };

    load(0, st[0]);
    if (1 < jend) {
        load(1, st[1]);
        wait_vmem_leave<ROUNDS>();
    } else {
        wait_vmem();
    }
    __syncthreads();
    // stage of tile j: j mod 3; tile j + 2 goes to the stage tile j - 1 used
    int cur = 0, ahead = 2;
    for (int j = 0; j < jend; ++j) {
        step(j, st[cur], st[ahead]);
        cur = cur == 2 ? 0 : cur + 1;
        ahead = ahead == 2 ? 0 : ahead + 1;
    }
    // position p = QPW w + 16 mb + 4 g + r  ->  query 64 mb + 16 g + 4 w + r
    float* out = dQ + head + (size_t)(i * BQ) * D;
#pragma unroll
    for (int mb = 0; mb < MBq; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int qrow = 64 * mb + 16 * g + 4 * w + r;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) out[(size_t)qrow * D + 16 * nb + n16] = acc[mb][nb][r];
        }
}

// Device pointers of one sage_bwd call.
struct BwdPtrs {
    const sage_qtensors* qk;
    const sage_dotensors* dos;
    const u16* V;    // 16-bit V, row-major
    const u16* dO;   // 16-bit dO, row-major
    const float* L;
    int8_t* dsw;
    float* sds;
    float *dQ, *dK, *dV;
};

template <bool BF16, int D, int BQ, bool CAUSAL>
hipError_t bwd_dispatch(const Dims& d, const BwdPtrs& p, hipStream_t s) {
    const sage_qtensors& qk = *p.qk;
    const sage_dotensors& dos = *p.dos;
    const dim3 grid(((d.Tn() + 1) / 2) * d.BH());
    auto kern = d.fp8       ? (d.q_smooth ? bwd_kernel<BF16, D, BQ, CAUSAL, true, false, true>
                                          : bwd_kernel<BF16, D, BQ, CAUSAL, false, false, true>)
                : d.dp_int8 ? (d.q_smooth ? bwd_kernel<BF16, D, BQ, CAUSAL, true, true, false>
                                          : bwd_kernel<BF16, D, BQ, CAUSAL, false, true, false>)
                            : (d.q_smooth ? bwd_kernel<BF16, D, BQ, CAUSAL, true, false, false>
                                          : bwd_kernel<BF16, D, BQ, CAUSAL, false, false, false>);
    kern<<<grid, 512, 0, s>>>(qk.q, qk.sq, qk.k, qk.sk, p.V, qk.vr, qk.sv, qk.mu_q, qk.qk_bias, dos.delta,
                              dos.dot, dos.sdo, p.dO, dos.dor, p.L, p.dsw, p.sds, p.dK, p.dV, d.N, d.BH(), d.scale);
    auto dq = d.fp8 ? dq_kernel<D, BQ, CAUSAL, true> : dq_kernel<D, BQ, CAUSAL, false>;
    dq<<<dim3(d.Tm() * d.BH()), 256, 0, s>>>(p.dsw, p.sds, qk.k, qk.sk, p.dQ, d.N, d.BH(), d.scale);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t bwd_dispatch_bq(const Dims& d, const BwdPtrs& p, hipStream_t s) {
    if (d.bq == 128)
        return d.causal ? bwd_dispatch<BF16, D, 128, true>(d, p, s) : bwd_dispatch<BF16, D, 128, false>(d, p, s);
    return d.causal ? bwd_dispatch<BF16, D, 64, true>(d, p, s) : bwd_dispatch<BF16, D, 64, false>(d, p, s);
}

size_t total_tiles(const Dims& d) {
    if (d.bq == 128)
        return d.BH() * (d.causal ? tiles_per_head<128, true>(d.Tm(), d.Tn()) : tiles_per_head<128, false>(d.Tm(), d.Tn()));
    return d.BH() * (d.causal ? tiles_per_head<64, true>(d.Tm(), d.Tn()) : tiles_per_head<64, false>(d.Tm(), d.Tn()));
}

size_t codes_bytes(const Dims& d) { return (total_tiles(d) * (size_t)d.bq * 64 + 255) / 256 * 256; }

}  // namespace

size_t bwd_workspace_bytes(const Dims& d) { return codes_bytes(d) + total_tiles(d) * sizeof(float); }

hipError_t launch_bwd(const Dims& d, const sage_qtensors& qk, const sage_dotensors& dos, const void* V,
                      const void* dO, const float* L, void* workspace, float* dQ, float* dK, float* dV,
                      hipStream_t s) {
    int8_t* dsw = static_cast<int8_t*>(workspace);
    float* sds = reinterpret_cast<float*>(dsw + codes_bytes(d));
    const BwdPtrs p{&qk, &dos, static_cast<const u16*>(V), static_cast<const u16*>(dO), L, dsw, sds, dQ, dK, dV};
    if (d.bf16) return d.D == 128 ? bwd_dispatch_bq<true, 128>(d, p, s) : bwd_dispatch_bq<true, 64>(d, p, s);
    return d.D == 128 ? bwd_dispatch_bq<false, 128>(d, p, s) : bwd_dispatch_bq<false, 64>(d, p, s);
}

}  // namespace sage
