// Device-side helpers shared by the SageBwd kernels (gfx950 only).
//
// Matrix-instruction operand orders used throughout (wave64, lane l):
//   v_mfma_i32_16x16x64_i8 / v_mfma_f32_16x16x32_*: A row m = l%16, B column
//     n = l%16; lane group g = l/16 and byte/element e carry the contraction
//     index; result register j holds row 4*g+j, column l%16.
// A and B only have to agree on which (g, e) carries which contraction
// index, so a result tile can feed the next product straight from registers
// once the other operand is stored in the matching permuted order (the
// C64P layout of sage.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLog2e_d = 1.4426950408889634074;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_127 = 6.988684686772166f;  // log2(127)
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448), the largest E4M3 value

// ---------------------------------------------------------------- dtypes
template <bool BF16>
__device__ __forceinline__ float to_f32(u16 b) {
    if constexpr (BF16) {
        return __uint_as_float((uint32_t)b << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, b);
    }
}

template <bool BF16>
__device__ __forceinline__ u16 from_f32(float x) {
    if constexpr (BF16) {
        uint32_t u = __float_as_uint(x);
        if ((u & 0x7f800000u) == 0x7f800000u) return (u16)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
        u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even
        return (u16)(u >> 16);
    } else {
        return __builtin_bit_cast(u16, (_Float16)x);  // v_cvt_f16_f32: nearest even
    }
}

// ---------------------------------------------------------------- layouts
// Byte offset of element (row, col) inside a head for each code layout of
// sage.h.  D is the head dimension.
__device__ __forceinline__ int off_r32(int row, int col, int D) {
    return (row >> 5) * (32 * D) + (((col >> 4) * 32 + (row & 31)) << 4) + (col & 15);
}
// C64P: 64-row group, (g, e) -> in-group row 16*(e/4) + 4*g + e%4.
__device__ __forceinline__ int off_c64p(int row, int col, int D) {
    int r = row & 63;
    int g = (r >> 2) & 3;
    int e = ((r >> 4) << 2) | (r & 3);
    return (row >> 6) * (64 * D) + ((g * D + col) << 4) + e;
}
// 16-bit row tiles (the backward's dO stage): element offset of (row, col).
__device__ __forceinline__ int off_r16h(int row, int col, int D) {
    return (row >> 4) * (16 * D) + ((((col >> 3) << 4) + (row & 15)) << 3) + (col & 7);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
// Maximum over the wave of non-negative floats, without LDS: the float bits
// of non-negative values order like integers, so rows of 16 lanes reduce by
// DPP rotations and the four row results by readlane.  Uniform result.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    int x = __float_as_int(v);
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));  // row_ror:8
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false));  // row_ror:4
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false));  // row_ror:2
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false));  // row_ror:1
    const int a = max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
    const int b = max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48));
    return __int_as_float(max(a, b));
}
__device__ __forceinline__ double wave_sum_d(double v, int width) {
    for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Round-half-even float -> int8 code in [-127, 127] (v is already scaled).
__device__ __forceinline__ int code_i8(float v) {
    float r = rintf(v);
    r = fminf(fmaxf(r, -127.f), 127.f);
    return (int)r;
}
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 255) | ((uint32_t)(b & 255) << 8) | ((uint32_t)(c & 255) << 16) |
           ((uint32_t)(d & 255) << 24);
}

// ---------------------------------------------------------------- LDS
typedef int v2i __attribute__((ext_vector_type(2)));
#define SAGE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// ds_read_b64_tr_b8: the 16 lanes of each lane group supply eight bytes each;
// lanes 2k and 2k+1 together name row k (16 bytes) of an 8 x 16 byte matrix,
// and lane i receives column i (byte k of the result = row k, byte i).
__device__ __forceinline__ v2i lds_read_tr8(const int8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(const_cast<int8_t*>(p)));
}

// Asynchronous 16-byte copy global -> LDS: lane l's 16 bytes from src land at
// lds_wave + 16 * l (lds_wave must be the same for the whole wave).  Tracked
// by vmcnt only; wait with wait_vmem() before the barrier that publishes the
// data.  Issued from inline assembly on purpose: the compiler would otherwise
// wait for the copy before every later LDS read it cannot prove disjoint from
// the destination, which serialises the copy of the next tile with the work
// on the current one.  M0 (the LDS base of the copy) is saved and restored
// around it, so the compiler's view of M0 is unchanged.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_wave) {
    const unsigned off =
        (unsigned)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(lds_wave));
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(src)
        : "memory");
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector memory operations of this wave are in flight
// (they complete in issue order for this count): with N the copies of the
// newest tile, every older tile has landed.
template <int N>
__device__ __forceinline__ void wait_vmem_leave() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS byte address of a __shared__ object (the value M0 takes for a copy).
template <typename T>
__device__ __forceinline__ unsigned lds_addr(const T* p) {
    return (unsigned)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) T*)(p));
}
// The same copies issued in groups with one save and restore of M0 and
// wave-uniform addresses: copy c moves lane l's 16 bytes at src_c + voff_c
// (src_c uniform, held in scalar registers; voff_c the lane's byte offset,
// normally 16 l) to LDS bytes [lds_c + 16 l, lds_c + 16 l + 16).  The address arithmetic of a
// group is scalar, outside the vector instruction stream.
__device__ __forceinline__ void copy16x1_to_lds(const void* s0, unsigned l0, unsigned voff) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %2\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(l0), "s"(s0), "v"(voff)
        : "memory");
}
// copy16x1_to_lds with the non-temporal hint, for data read exactly once (the
// backward's dS workspace): its lines then leave L2 first and do not push out
// operands that other workgroups read again.
__device__ __forceinline__ void copy16x1_nt_to_lds(const void* s0, unsigned l0, unsigned voff) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %2 nt\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(l0), "s"(s0), "v"(voff)
        : "memory");
}
__device__ __forceinline__ void copy16x2_to_lds(const void* s0, unsigned l0, unsigned v0, const void* s1, unsigned l1,
                                                unsigned v1) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %3\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %4\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(l0), "s"(l1), "s"(s0), "s"(s1), "v"(v0), "v"(v1)
        : "memory");
}
__device__ __forceinline__ void copy16x4_to_lds(const void* s0, unsigned l0, unsigned v0, const void* s1, unsigned l1,
                                                unsigned v1, const void* s2, unsigned l2, unsigned v2,
                                                const void* s3, unsigned l3, unsigned v3) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, %5\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %10, %6\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %11, %7\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %12, %8\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(l0), "s"(l1), "s"(l2), "s"(l3), "s"(s0), "s"(s1), "s"(s2), "s"(s3), "v"(v0), "v"(v1), "v"(v2),
          "v"(v3)
        : "memory");
}
// Copies of rounds [0, N) given as (source, LDS address, lane offset)
// lists, four, two or one per statement.
template <int N>
__device__ __forceinline__ void copy16_rounds(const int8_t* const* src, const unsigned* dst, const unsigned* vo) {
    int u = 0;
#pragma unroll
    for (; u + 4 <= N; u += 4)
        copy16x4_to_lds(src[u], dst[u], vo[u], src[u + 1], dst[u + 1], vo[u + 1], src[u + 2], dst[u + 2], vo[u + 2],
                        src[u + 3], dst[u + 3], vo[u + 3]);
    if constexpr (N % 4 >= 2) {
        constexpr int b = N / 4 * 4;
        copy16x2_to_lds(src[b], dst[b], vo[b], src[b + 1], dst[b + 1], vo[b + 1]);
    }
    if constexpr (N % 2 == 1) copy16x1_to_lds(src[N - 1], dst[N - 1], vo[N - 1]);
}
// The compiler does not count the copies above either, so a register loaded
// from global memory before some copies and first used after them would get
// its wait at the use, where that wait (vmcnt counts in issue order) also
// waits for every copy issued in between.  settle() right after wait_vmem()
// makes the compiler take its wait for the register there instead, where it
// costs nothing.
template <typename T>
__device__ __forceinline__ void settle(T& x) { asm volatile("" : "+v"(x)); }

// ---------------------------------------------------------------- MFMA
// Integer products with a float conversion for free: an int32 accumulator
// started at the bits of 1.5 * 2^23 holds, read as a float, exactly
// 1.5 * 2^23 + sum while |sum| < 2^22 (every product here has
// |sum| <= 127 * 127 * 128 < 2^21), so one exact subtraction recovers it.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagicF = 12582912.0f;
__device__ __forceinline__ float unmagic(int x) { return __int_as_float(x) - kMagicF; }

__device__ __forceinline__ v4i mfma16_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// E4M3 products with float32 accumulation, on the same 16-byte operand chunks
// (lane group g, byte e) as the INT8 product.  v_mfma_f32_16x16x32_fp8_fp8
// contracts 8 bytes per lane, so two of them cover a chunk (bytes 0-7, then
// 8-15).  v_mfma_f32_16x16x128_f8f6f4 (format 0 = E4M3 for both operands, no
// block scale) contracts 32 bytes per lane: two chunks at once.  In both, A
// and B pair the same (g, byte) positions, which is all a contraction needs.
typedef int v8i __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mfma16_f8x64(v4i a, v4i b, v4f c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, v2i{a[0], a[1]}),
                                                   __builtin_bit_cast(long, v2i{b[0], b[1]}), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, v2i{a[2], a[3]}),
                                                      __builtin_bit_cast(long, v2i{b[2], b[3]}), c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma16_f8x128(v4i a0, v4i a1, v4i b0, v4i b1, v4f c) {
    const v8i a = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const v8i b = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// Float value of one accumulator element: INT8 (magic-started int32) or E4M3
// (float32).
__device__ __forceinline__ float acc_value(int x) { return unmagic(x); }
__device__ __forceinline__ float acc_value(float x) { return x; }
// Four E4M3 codes (nearest value, ties to even) packed into bytes 0..3.
__device__ __forceinline__ int pack_e4m3(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
template <bool BF16>
__device__ __forceinline__ v4f mfma16_h(v4i a, v4i b, v4f c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                       __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                      __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    }
}

}  // namespace sage
