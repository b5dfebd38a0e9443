// Device-side helpers shared by the PASA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace pasa {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, fp16) * B(16x32, fp16) on the matrix cores.
// Lane l supplies A row (l % 32), B column (l % 32), and 8 consecutive
// contraction slots starting at 8 * (l / 32); it receives D column (l % 32),
// rows 8 * (r / 4) + 4 * (l / 32) + (r % 4) for r = 0..15.
__device__ __forceinline__ f16v mfma_32x32x16(h8 a, h8 b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Reductions across the two halves of the wave (lanes l and l^32).
// v_permlane32_swap(x, x) yields (x[l], x[l+32]) in lanes 0-31 and
// (x[l-32], x[l]) in lanes 32-63, so combining its two results in that order
// gives both lanes of a pair the identical, order-fixed value.
__device__ __forceinline__ float xsum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// max of three floats in one instruction; no NaN canonicalisation of the
// inputs (the kernels feed it finite scores and -inf).  It is inline assembly,
// and the compiler's hazard recognizer does not look into inline assembly: a
// read of a matrix product's result needs wait states after the product
// (the compiler puts s_nop 11 before its own vector read of a 32x32x16
// result), so where a product's result may reach max3f with no other
// products issued in between, the caller passes it through xdl_fence first.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float xmax32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return m;
}
__device__ __forceinline__ _Float16 xsum32(_Float16 x) {
    const unsigned u = __builtin_bit_cast(unsigned short, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(_Float16, (unsigned short)r[0]) +
           __builtin_bit_cast(_Float16, (unsigned short)r[1]);
}
__device__ __forceinline__ _Float16 xmax32(_Float16 x) {
    const unsigned u = __builtin_bit_cast(unsigned short, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const _Float16 a = __builtin_bit_cast(_Float16, (unsigned short)r[0]);
    const _Float16 b = __builtin_bit_cast(_Float16, (unsigned short)r[1]);
    return a > b ? a : b;
}

// Orders every later read of x after 24 wait states (three s_nop 7): the
// asm takes x as an in/out operand, so the compiler issues it after the
// product that writes x and every use of x after it.  24 covers the compiler's
// own 12 for a 32x32x16 fp16 result with room for the longer fp8 product.
__device__ __forceinline__ void xdl_fence(f16v& x) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}

__device__ __forceinline__ bool wave_any(bool p) {
    return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ _Float16 hexp2(_Float16 x) { return __builtin_elementwise_exp2(x); }

__device__ __forceinline__ h2 hmax(h2 a, h2 b) { return __builtin_elementwise_max(a, b); }

// exp2 of both halves of four packed pairs, in place (same registers, no
// repacking): the SDWA form of v_exp_f16 on the low halves, preserving the
// high halves, then on the high halves, preserving the low results.  A
// preserving write reads the register a transcendental instruction just
// wrote.  The CDNA instruction-set guides' table of manually inserted wait
// states asks for one wait state after a transcendental op whose result a
// non-transcendental VALU op reads, and one after a sub-dword SDWA write
// whose register a VALU op reads; the compiler's hazard recognizer does not
// see inside inline asm.  Issuing the four low halves first puts three
// instructions between each pair, and the trailing s_nop 1 (two wait states)
// separates the last write from the first consumer after the block.
__device__ __forceinline__ void hexp2_pk4(h2* r) {
    asm("v_exp_f16_sdwa %0, %0 dst_sel:WORD_0 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0\n\t"
        "v_exp_f16_sdwa %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0\n\t"
        "v_exp_f16_sdwa %2, %2 dst_sel:WORD_0 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0\n\t"
        "v_exp_f16_sdwa %3, %3 dst_sel:WORD_0 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0\n\t"
        "v_exp_f16_sdwa %0, %0 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1\n\t"
        "v_exp_f16_sdwa %1, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1\n\t"
        "v_exp_f16_sdwa %2, %2 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1\n\t"
        "v_exp_f16_sdwa %3, %3 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1\n\t"
        "s_nop 1"
        : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
}

// hexp2_pk4 for two pairs, kept after the instruction that produced `after`.
// The asm names `after` as an input and never reads it, so the compiler
// cannot hoist the exponentials above that instruction; a scheduling fence
// alone does not stop it.  One instruction separates the two writes to each
// register, which is the one wait state that both hazards above ask for.
__device__ __forceinline__ void hexp2_pk2_after(h2* r, const f16v& after) {
    asm volatile("v_exp_f16_sdwa %0, %0 dst_sel:WORD_0 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0\n\t"
                 "v_exp_f16_sdwa %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0\n\t"
                 "v_exp_f16_sdwa %0, %0 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1\n\t"
                 "v_exp_f16_sdwa %1, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1\n\t"
                 "s_nop 1"
                 : "+v"(r[0]), "+v"(r[1])
                 : "v"(after));
}

// f(std::integral_constant<int, i>{}) for i = B .. E-1, unrolled at compile
// time, so that the body sees i as a constant expression.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// fp16(c * a + z) for fp32 operands with one rounding (fused multiply-add in
// mixed precision, round-to-nearest-even).
__device__ __forceinline__ _Float16 fma_to_h(float a, float c, float z) {
    h2 t;
    asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]" : "=v"(t) : "v"(a), "v"(c), "v"(z));
    return t.x;
}

// Two floats rounded to fp16 (round-to-nearest-even) and packed.
__device__ __forceinline__ h2 to_h2(float a, float b) {
    return __builtin_convertvector((float __attribute__((ext_vector_type(2)))){a, b}, h2);
}

constexpr _Float16 kHalfNegInf = -__builtin_inff16();

}  // namespace pasa
