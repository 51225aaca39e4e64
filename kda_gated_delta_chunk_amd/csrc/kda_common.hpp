// Shared device helpers for the gfx950 KDA kernels: bf16 packing, MFMA
// fragment types and the two matrix-core products every kernel uses.
//
// Matrix-core layout used throughout (one 64-lane wavefront, 16x16 output):
//   accumulator / D tile : lane l holds D[4*(l/16) + i][l%16], i = 0..3
//   mma16 operands       : lane l holds A[l%16][4*(l/16) + i] and
//                          B[4*(l/16) + i][l%16], i = 0..3 (16-deep product)
//   mma32 operands       : lane l holds 8 reduction slots, slot j <-> reduction
//                          index 8*(l/16) + j, the same map for A and B
//                          (32-deep product). Any bijection between slots and
//                          reduction indices gives the same sum as long as A
//                          and B agree; the kernels pick the map that lets an
//                          accumulator tile pair feed a product directly.
// A 16-deep accumulator tile therefore IS a valid B operand of mma16, which is
// what lets the inter-chunk state and the corrected values stay in registers.
//
// Two element types share one code path:
//   bf16 I/O : operands are bf16 (bit patterns in uint32 pairs), products run
//              on v_mfma_f32_16x16x16_bf16 / v_mfma_f32_16x16x32_bf16 with fp32
//              accumulation;
//   fp32 I/O : operands are fp32, every product runs as a sum of
//              v_mfma_f32_16x16x4_f32 steps (step i takes slot i of each lane,
//              which realises the same slot map as above).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round two floats to bf16 (round-to-nearest-even, one v_cvt_pk_bf16_f32) and pack (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 p;
    p[0] = (__bf16)a;
    p[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, p);
}

// Split x into hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits in two bf16s.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pack_bf16(a, b);
    lo = pack_bf16(a - bf_lo(hi), b - bf_hi(hi));
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// Round two floats to fp16 (round-to-nearest-even) and pack (a in the low half).
__device__ __forceinline__ uint32_t pack_h(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) _Float16 h2;
    h2 p;
    p[0] = (_Float16)a;
    p[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, p);
}

// ------------------------------------------------------------ fragment types
// Frag4: 4 reduction slots per lane (mma16 operand). Frag8: 8 slots (mma32 operand).
template <bool BF> struct Frag4;
template <> struct Frag4<true> { uint32_t p[2]; };   // 4 bf16
template <> struct Frag4<false> { float f[4]; };     // 4 fp32
template <bool BF> struct Frag8;
template <> struct Frag8<true> { uint32_t p[4]; };   // 8 bf16
template <> struct Frag8<false> { float f[8]; };     // 8 fp32

// Build operands from fp32 values (bf16: rounded to nearest even).
__device__ __forceinline__ void set4(Frag4<true> &a, float x0, float x1, float x2, float x3) {
    a.p[0] = pack_bf16(x0, x1);
    a.p[1] = pack_bf16(x2, x3);
}
__device__ __forceinline__ void set4(Frag4<false> &a, float x0, float x1, float x2, float x3) {
    a.f[0] = x0; a.f[1] = x1; a.f[2] = x2; a.f[3] = x3;
}

// D += A * B, 16 x 16 x 16.
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const Frag4<true> &a, const Frag4<true> &b) {
    s16x4 av = __builtin_bit_cast(s16x4, make_uint2(a.p[0], a.p[1]));
    s16x4 bv = __builtin_bit_cast(s16x4, make_uint2(b.p[0], b.p[1]));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const Frag4<false> &a, const Frag4<false> &b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[i], b.f[i], acc, 0, 0, 0);
    return acc;
}
// D += A * B, 16 x 16 x 32.
__device__ __forceinline__ f32x4 mma32(f32x4 acc, const Frag8<true> &a, const Frag8<true> &b) {
    bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(a.p[0], a.p[1], a.p[2], a.p[3]));
    bf16x8 bv = __builtin_bit_cast(bf16x8, make_uint4(b.p[0], b.p[1], b.p[2], b.p[3]));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(f32x4 acc, const Frag8<false> &a, const Frag8<false> &b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[i], b.f[i], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Explicit wait states between matrix-core products and the first
// non-matrix-core instruction that reads their results (VALU, accumulator
// read, LDS or global store). On gfx950 the compiler's own padding after a
// bf16 16x16x16 product (8 wait states) has been observed to be too short: the
// first elements read back (rows 4g and 4g+1 of the tile) came out stale. The
// padding is an asm statement that takes the results as read-write VGPR
// operands (the kernels keep accumulators in VGPRs: their register budget is at
// most 256 per lane), so every consumer depends on it, every producing product
// precedes it, and no copy of the results is placed in front of the padding. (A scheduling barrier
// alone does not stop the compiler from sinking a pure product below it.)
__device__ __forceinline__ void mfma_fence(f32x4 &a) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a));
}
__device__ __forceinline__ void mfma_fence(f32x4 &a, f32x4 &b) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void mfma_fence(f32x4 &a, f32x4 &b, f32x4 &c) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c));
}
__device__ __forceinline__ void mfma_fence(f32x4 &a, f32x4 &b, f32x4 &c, f32x4 &d) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void mfma_fence(f32x4 &a, f32x4 &b, f32x4 &c, f32x4 &d, f32x4 &e) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e));
}
__device__ __forceinline__ void mfma_fence(f32x4 &a, f32x4 &b, f32x4 &c, f32x4 &d, f32x4 &e, f32x4 &f) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f));
}
// The same for a whole register tile of the state (2, 4 or 8 accumulators),
// in one asm statement so that the padding sits between every product and its
// readers.
__device__ __forceinline__ void mfma_fence_all(f32x4 (&x)[2]) { mfma_fence(x[0], x[1]); }
__device__ __forceinline__ void mfma_fence_all(f32x4 (&x)[4]) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}
__device__ __forceinline__ void mfma_fence_all(f32x4 (&x)[8]) {
    asm volatile("s_nop 7\n\ts_nop 7"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
}

// Cross-lane moves inside a 16-lane row (DPP). row_scan16 is the inclusive
// prefix sum over the 16 lanes of each row; row_suffix16 the exclusive suffix
// sum; row_last broadcasts lane 15 of each row to the whole row.
template <int CTRL, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                                 BOUND_ZERO));
}
__device__ __forceinline__ float row_scan16(float x) {
    x += dpp_f<0x111, true>(x);  // row_shr:1, lanes without a source add 0
    x += dpp_f<0x112, true>(x);  // row_shr:2
    x += dpp_f<0x114, true>(x);  // row_shr:4
    x += dpp_f<0x118, true>(x);  // row_shr:8
    return x;
}
// Exclusive suffix sum over the 16 lanes of each row: lane r gets the sum of lanes r+1 .. 15 (0 on lane 15).
// A decay exponent spanning tokens r+1 .. 15 is summed from those tokens' own terms: formed as the row total
// minus the inclusive prefix it would carry an error of the total's size, not of its own.
__device__ __forceinline__ float row_suffix16(float x) {
    x = dpp_f<0x101, true>(x);   // row_shl:1, lane 15 has no source and takes 0
    x += dpp_f<0x101, true>(x);  // row_shl:1
    x += dpp_f<0x102, true>(x);  // row_shl:2
    x += dpp_f<0x104, true>(x);  // row_shl:4
    x += dpp_f<0x108, true>(x);  // row_shl:8
    return x;
}
__device__ __forceinline__ float row_last(float x) { return dpp_f<0x15f, true>(x); }  // row_newbcast:15
// Lane k of each 16-lane row, broadcast to the row (row_newbcast:k); k must be a compile-time constant.
__device__ __forceinline__ float row_bcast(float x, int k) {
    switch (k) {
        case 0: return dpp_f<0x150, true>(x);
        case 1: return dpp_f<0x151, true>(x);
        case 2: return dpp_f<0x152, true>(x);
        case 3: return dpp_f<0x153, true>(x);
        case 4: return dpp_f<0x154, true>(x);
        case 5: return dpp_f<0x155, true>(x);
        case 6: return dpp_f<0x156, true>(x);
        case 7: return dpp_f<0x157, true>(x);
        case 8: return dpp_f<0x158, true>(x);
        case 9: return dpp_f<0x159, true>(x);
        case 10: return dpp_f<0x15a, true>(x);
        case 11: return dpp_f<0x15b, true>(x);
        case 12: return dpp_f<0x15c, true>(x);
        case 13: return dpp_f<0x15d, true>(x);
        case 14: return dpp_f<0x15e, true>(x);
        default: return dpp_f<0x15f, true>(x);
    }
}

// Two column tiles of the state (2 x 2, 2 x 4 or 2 x 8 accumulators), one asm statement.
__device__ __forceinline__ void mfma_fence_all(f32x4 (&x)[2][2]) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[1][0]), "+v"(x[1][1]));
}
__device__ __forceinline__ void mfma_fence_all(f32x4 (&x)[2][4]) {
    asm volatile("s_nop 7\n\ts_nop 7"
                 : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[1][0]), "+v"(x[1][1]),
                   "+v"(x[1][2]), "+v"(x[1][3]));
}
__device__ __forceinline__ void mfma_fence_all(f32x4 (&x)[2][8]) {
    asm volatile("s_nop 7\n\ts_nop 7"
                 : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[0][4]), "+v"(x[0][5]),
                   "+v"(x[0][6]), "+v"(x[0][7]), "+v"(x[1][0]), "+v"(x[1][1]), "+v"(x[1][2]), "+v"(x[1][3]),
                   "+v"(x[1][4]), "+v"(x[1][5]), "+v"(x[1][6]), "+v"(x[1][7]));
}

template <int N> __device__ __forceinline__ void mfma_fence_all(f32x4 (&x)[1][N]) { mfma_fence_all(x[0]); }

// e^x through the hardware base-2 exponential.
__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// The bounded log-decay gate of "Kimi K3 发布核实与 Moonshot AI 主干架构演变" (section 3,
// paragraph "K3 对 Kimi Linear 的进一步修改"): a sigmoid of the pre-activation x scaled so the
// log-decay lies in (-5, 0), returned in base 2 (log2 of the retention):
//   -5 log2(e) / (1 + e^-x).
// For x below about -88 the exponential overflows to +inf and the result is -0 (no decay); for
// large x it tends to -5 log2(e). v_exp_f32 and v_rcp_f32 are each within 1 ulp.
__device__ __forceinline__ float gate_log2_decay(float x) {
    constexpr float L2E = 1.4426950408889634f;
    return (-5.f * L2E) * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * L2E));
}

// 1 / (1 + e^-x) in fp32 (the output gate's activation); exactly 0 below about -88, 1 for large x.
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// fp16 operands (Frag4<true> / Frag8<true> holding fp16 bit pairs instead of bf16): D += A * B on
// v_mfma_f32_16x16x16_f16 / v_mfma_f32_16x16x32_f16, with the same lane and slot layout as mma16 /
// mma32.
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
__device__ __forceinline__ f32x4 mmah16(f32x4 acc, const Frag4<true> &a, const Frag4<true> &b) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, make_uint2(a.p[0], a.p[1])),
                                                 __builtin_bit_cast(f16x4, make_uint2(b.p[0], b.p[1])), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mmah32(f32x4 acc, const Frag8<true> &a, const Frag8<true> &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(f16x8, make_uint4(a.p[0], a.p[1], a.p[2], a.p[3])),
        __builtin_bit_cast(f16x8, make_uint4(b.p[0], b.p[1], b.p[2], b.p[3])), acc, 0, 0, 0);
}

// I/O element access by dtype.
template <bool BF> struct IO;
template <> struct IO<true> {
    using T = uint16_t;
    static __device__ __forceinline__ float ld(const T *p, int64_t i) { return bf2f(p[i]); }
    static __device__ __forceinline__ void st(T *p, int64_t i, float x) {
        bf16x2 v;
        v[0] = (__bf16)x;
        p[i] = __builtin_bit_cast(uint16_t, v[0]);
    }
};
template <> struct IO<false> {
    using T = float;
    static __device__ __forceinline__ float ld(const T *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(T *p, int64_t i, float x) { p[i] = x; }
};

}  // namespace kda
