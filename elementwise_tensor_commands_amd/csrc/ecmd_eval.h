// ecmd_eval.h -- per-element evaluation of a lowered Program on gfx950.
//
// Values are 32-bit containers: binary32 bits, int32, or binary16 bits in the
// low half.  Each work-item evaluates E consecutive elements at once.
//
// Two evaluators share the operation semantics below:
//   * RtEval interprets the Program held in the kernel argument block.  Every
//     branch depends only on Program bytes, which are the same for all lanes,
//     so the wavefront never diverges.  Operands are picked by switch
//     statements over compile-time register names: the register file stays in
//     VGPRs (a runtime-indexed private array would live in scratch memory).
//   * CtEval<P> evaluates a compile-time Program: the operation list is
//     unrolled by template recursion and every reference is a constant, so the
//     code is what one would write by hand for that Command.
//
// This file must be compiled with -ffp-contract=off: each binary32 operation
// rounds on its own, as the E_ operations are separate operations of the
// Command (rocRoller "Design Overview", section "Operations").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ecmd_tape.h"

namespace ecmd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// binary16 -> binary32 (exact; v_cvt_f32_f16 keeps subnormals in FP16 denorm mode 3).
__device__ __forceinline__ uint32_t h2f(uint32_t h)
{
    _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)h);
    return as_u((float)x);
}

// binary32 -> binary16, round to nearest even (v_cvt_f16_f32 under the default
// round mode), overflow to infinity, gradual underflow.  The empty asm pins the
// binary32 operand in a VGPR: without it the backend folds a preceding binary32
// multiply into the conversion (v_fma_mix* with a +0 addend), which rounds the
// exact product once instead of twice and turns a -0 product into +0.
__device__ __forceinline__ uint32_t f2h(uint32_t f)
{
    float v = as_f(f);
    asm("" : "+v"(v));
    _Float16 x = (_Float16)v;
    return (uint32_t)__builtin_bit_cast(uint16_t, x);
}

// bfloat16 -> binary32: the 16 bits are binary32's upper half (exact).
__device__ __forceinline__ uint32_t bf2f(uint32_t h) { return h << 16; }

// binary32 -> bfloat16: gfx950 converts in one instruction (v_cvt_pk_bf16_f32,
// two values per instruction), rounding to nearest even under the default
// round mode, with binary32 subnormals kept (FP32 denorm mode 3) and NaN kept
// NaN.  The GPU tests compare it with the oracle on all 2^32 patterns.
__device__ __forceinline__ uint32_t f2bf(uint32_t f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)as_f(f));
}

// int32 -> bfloat16, rounded once from the exact integer (through binary32
// would round twice: 2^24 + 2^16 + 1 would land on a midpoint).  |a| is
// shifted to an 8-bit significand; the dropped bits decide the rounding.
// Selects only (see minmax16).
__device__ __forceinline__ uint32_t i2bf(uint32_t a)
{
    const uint32_t sign = (a >> 16) & 0x8000u;
    const uint32_t m = (a & 0x80000000u) ? 0u - a : a;      // |INT_MIN| = 2^31 as unsigned
    uint32_t e = 31u - (uint32_t)__builtin_clz(m | 1u);      // leading bit position (m = 0: handled last)
    const uint32_t sh = e > 7u ? e - 7u : 0u;                // bits dropped below the 8-bit significand
    uint32_t q = (m >> sh) << (e > 7u ? 0u : 7u - e);
    const uint32_t rem = m & ((1u << sh) - 1u), half = sh ? 1u << ((sh - 1u) & 31u) : 0u;
    q += (sh != 0u && (rem > half || (rem == half && (q & 1u)))) ? 1u : 0u;
    const bool carry = q == 256u;                            // carried into the next binade
    q = carry ? 128u : q;
    e += carry ? 1u : 0u;
    return m == 0u ? 0u : sign | ((e + 127u) << 7) | (q & 0x7fu);
}

// Value of a binary16 / bfloat16 pattern as binary32 bits (exact).
template <bool BF>
__device__ __forceinline__ uint32_t h16f(uint32_t h) { return BF ? bf2f(h) : h2f(h); }

// binary16 / bfloat16 minimum and maximum on the exact values; the result is
// one operand's 16-bit pattern (NaN operand ignored unless both are, -0 below
// +0).  Selects only, no early returns: a return per case compiles to branches
// that differ between lanes (exec-mask juggling for every element).
template <bool BF, bool MAX>
__device__ __forceinline__ uint32_t minmax16(uint32_t a, uint32_t b)
{
    const float x = as_f(h16f<BF>(a)), y = as_f(h16f<BF>(b));
    const bool a_neg = (a & 0x8000u) != 0u;
    uint32_t r = (MAX ? x > y : x < y) ? a : b;
    r = (x == y) ? ((MAX ? !a_neg : a_neg) ? a : b) : r;
    r = (y != y) ? a : r;
    return (x != x) ? b : r;
}

// binary16 arithmetic in the format itself (v_add_f16 and friends: one IEEE
// rounding, binary16 subnormals kept in FP16 denorm mode 3).
__device__ __forceinline__ _Float16 as_h(uint32_t u) { return __builtin_bit_cast(_Float16, (uint16_t)u); }
__device__ __forceinline__ uint32_t h_bits(_Float16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

// binary32 -> int32: truncate toward zero, saturate, NaN -> 0.  Written out so
// that no out-of-range conversion (undefined in C++) is ever performed, with
// selects rather than early returns (see minmax16).
__device__ __forceinline__ uint32_t f2i_sat(float f)
{
    const bool hi = f >= 2147483648.0f, lo = f < -2147483648.0f, nan = !(f == f);
    const float in_range = (hi || lo || nan) ? 0.0f : f;
    uint32_t r = (uint32_t)(int32_t)in_range;
    r = hi ? 0x7fffffffu : r;
    return lo ? 0x80000000u : r;
}

// binary32 minimum / maximum: a NaN operand is ignored unless both are NaN;
// -0 is below +0.  Written with comparisons and selects, not v_min/v_max, so
// that the result does not depend on the hardware's NaN and signed-zero rules
// (and with selects only, see minmax16).
__device__ __forceinline__ uint32_t fmin_bits(uint32_t a, uint32_t b)
{
    const float x = as_f(a), y = as_f(b);
    uint32_t r = x < y ? a : b;
    r = (x == y) ? ((a & 0x80000000u) ? a : b) : r;
    r = (y != y) ? a : r;
    return (x != x) ? b : r;
}

__device__ __forceinline__ uint32_t fmax_bits(uint32_t a, uint32_t b)
{
    const float x = as_f(a), y = as_f(b);
    uint32_t r = x > y ? a : b;
    r = (x == y) ? ((a & 0x80000000u) ? b : a) : r;
    r = (y != y) ? a : r;
    return (x != x) ? b : r;
}

template <int C>
__device__ __forceinline__ uint32_t apply(uint32_t a, uint32_t b, uint32_t c = 0u)
{
    if constexpr (C == C_MOV) return a;
    else if constexpr (C == C_ADD_F32) return as_u(as_f(a) + as_f(b));
    else if constexpr (C == C_SUB_F32) return as_u(as_f(a) - as_f(b));
    else if constexpr (C == C_MUL_F32) return as_u(as_f(a) * as_f(b));
    else if constexpr (C == C_ADD_I32) return a + b;
    else if constexpr (C == C_SUB_I32) return a - b;
    else if constexpr (C == C_MUL_I32) return a * b;
    else if constexpr (C == C_NEG_F32) return a ^ 0x80000000u;
    else if constexpr (C == C_NEG_I32) return 0u - a;
    else if constexpr (C == C_NEG_F16) return (a ^ 0x8000u) & 0xffffu;
    else if constexpr (C == C_CVT_F16_F32) return h2f(a);
    else if constexpr (C == C_CVT_F32_F16) return f2h(a);
    else if constexpr (C == C_CVT_I32_F32) return as_u((float)(int32_t)a);
    else if constexpr (C == C_CVT_F32_I32) return f2i_sat(as_f(a));
    // int32 -> binary16 through binary32: exact below 2^24, and at or above
    // 2^24 both this and a direct rounding give infinity, so one rounding.
    else if constexpr (C == C_CVT_I32_F16) return f2h(as_u((float)(int32_t)a));
    else if constexpr (C == C_CVT_F16_I32) return f2i_sat(as_f(h2f(a)));
    else if constexpr (C == C_EQ_F32) return as_f(a) == as_f(b) ? 1u : 0u;
    else if constexpr (C == C_NE_F32) return as_f(a) != as_f(b) ? 1u : 0u;
    else if constexpr (C == C_LT_F32) return as_f(a) < as_f(b) ? 1u : 0u;
    else if constexpr (C == C_LE_F32) return as_f(a) <= as_f(b) ? 1u : 0u;
    else if constexpr (C == C_GT_F32) return as_f(a) > as_f(b) ? 1u : 0u;
    else if constexpr (C == C_GE_F32) return as_f(a) >= as_f(b) ? 1u : 0u;
    else if constexpr (C == C_EQ_I32) return a == b ? 1u : 0u;
    else if constexpr (C == C_NE_I32) return a != b ? 1u : 0u;
    else if constexpr (C == C_LT_I32) return (int32_t)a < (int32_t)b ? 1u : 0u;
    else if constexpr (C == C_LE_I32) return (int32_t)a <= (int32_t)b ? 1u : 0u;
    else if constexpr (C == C_GT_I32) return (int32_t)a > (int32_t)b ? 1u : 0u;
    else if constexpr (C == C_GE_I32) return (int32_t)a >= (int32_t)b ? 1u : 0u;
    else if constexpr (C == C_LT_U32) return a < b ? 1u : 0u;
    else if constexpr (C == C_LE_U32) return a <= b ? 1u : 0u;
    else if constexpr (C == C_GT_U32) return a > b ? 1u : 0u;
    else if constexpr (C == C_GE_U32) return a >= b ? 1u : 0u;
    else if constexpr (C == C_MIN_F32) return fmin_bits(a, b);
    else if constexpr (C == C_MAX_F32) return fmax_bits(a, b);
    else if constexpr (C == C_MIN_I32) return (int32_t)a < (int32_t)b ? a : b;
    else if constexpr (C == C_MAX_I32) return (int32_t)a > (int32_t)b ? a : b;
    else if constexpr (C == C_ABS_F32) return a & 0x7fffffffu;
    else if constexpr (C == C_ABS_I32) return (a & 0x80000000u) ? 0u - a : a;
    else if constexpr (C == C_ABS_F16) return a & 0x7fffu;
    else if constexpr (C == C_SELECT) return a != 0u ? b : c;
    else if constexpr (C == C_ADD_F16) return h_bits(as_h(a) + as_h(b));
    else if constexpr (C == C_SUB_F16) return h_bits(as_h(a) - as_h(b));
    else if constexpr (C == C_MUL_F16) return h_bits(as_h(a) * as_h(b));
    // bfloat16 arithmetic through binary32: the binary32 result of two
    // bfloat16 operands, rounded to bfloat16, equals the exact result rounded
    // once (24 >= 2*8 + 2 bits; Figueroa 1995).
    else if constexpr (C == C_ADD_BF16) return f2bf(as_u(as_f(bf2f(a)) + as_f(bf2f(b))));
    else if constexpr (C == C_SUB_BF16) return f2bf(as_u(as_f(bf2f(a)) - as_f(bf2f(b))));
    else if constexpr (C == C_MUL_BF16) return f2bf(as_u(as_f(bf2f(a)) * as_f(bf2f(b))));
    else if constexpr (C == C_NEG_BF16) return (a ^ 0x8000u) & 0xffffu;
    else if constexpr (C == C_ABS_BF16) return a & 0x7fffu;
    else if constexpr (C == C_CVT_F16_BF16) return f2bf(h2f(a));
    else if constexpr (C == C_CVT_BF16_F16) return f2h(bf2f(a));
    else if constexpr (C == C_CVT_BF16_F32) return bf2f(a);
    else if constexpr (C == C_CVT_F32_BF16) return f2bf(a);
    else if constexpr (C == C_CVT_BF16_I32) return f2i_sat(as_f(bf2f(a)));
    else if constexpr (C == C_CVT_I32_BF16) return i2bf(a);
    else if constexpr (C == C_EQ_F16) return as_f(h2f(a)) == as_f(h2f(b)) ? 1u : 0u;
    else if constexpr (C == C_NE_F16) return as_f(h2f(a)) != as_f(h2f(b)) ? 1u : 0u;
    else if constexpr (C == C_LT_F16) return as_f(h2f(a)) < as_f(h2f(b)) ? 1u : 0u;
    else if constexpr (C == C_LE_F16) return as_f(h2f(a)) <= as_f(h2f(b)) ? 1u : 0u;
    else if constexpr (C == C_GT_F16) return as_f(h2f(a)) > as_f(h2f(b)) ? 1u : 0u;
    else if constexpr (C == C_GE_F16) return as_f(h2f(a)) >= as_f(h2f(b)) ? 1u : 0u;
    else if constexpr (C == C_EQ_BF16) return as_f(bf2f(a)) == as_f(bf2f(b)) ? 1u : 0u;
    else if constexpr (C == C_NE_BF16) return as_f(bf2f(a)) != as_f(bf2f(b)) ? 1u : 0u;
    else if constexpr (C == C_LT_BF16) return as_f(bf2f(a)) < as_f(bf2f(b)) ? 1u : 0u;
    else if constexpr (C == C_LE_BF16) return as_f(bf2f(a)) <= as_f(bf2f(b)) ? 1u : 0u;
    else if constexpr (C == C_GT_BF16) return as_f(bf2f(a)) > as_f(bf2f(b)) ? 1u : 0u;
    else if constexpr (C == C_GE_BF16) return as_f(bf2f(a)) >= as_f(bf2f(b)) ? 1u : 0u;
    else if constexpr (C == C_MIN_F16) return minmax16<false, false>(a, b);
    else if constexpr (C == C_MAX_F16) return minmax16<false, true>(a, b);
    else if constexpr (C == C_MIN_BF16) return minmax16<true, false>(a, b);
    else if constexpr (C == C_MAX_BF16) return minmax16<true, true>(a, b);
    else return 0u;
}

// n / d for a 32-bit n, by the multiplier and shifts of FastDiv.
__device__ __forceinline__ uint32_t fast_div(const FastDiv &f, uint32_t n)
{
    const uint32_t t = __umulhi(n, f.mul);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

// ---------------------------------------------------------------------------
// Generic interpreter.

template <int E>
struct Regs {
    uint32_t in[kMaxIn][E];
    uint32_t s[kMaxSlot][E];
};

template <int E>
__device__ __forceinline__ void rt_fetch(uint8_t ref, const Regs<E> &R, const uint32_t *uni,
                                         uint32_t (&o)[E])
{
    switch (ref) {
#define ECMD_FETCH_IN(k)                                  \
    case kRefIn + k:                                      \
        _Pragma("unroll") for (int e = 0; e < E; ++e) o[e] = R.in[k][e]; \
        break;
#define ECMD_FETCH_S(k)                                   \
    case kRefSlot + k:                                    \
        _Pragma("unroll") for (int e = 0; e < E; ++e) o[e] = R.s[k][e]; \
        break;
#define ECMD_FETCH_U(k)                                   \
    case kRefUni + k: {                                   \
        const uint32_t u = uni[k];                        \
        _Pragma("unroll") for (int e = 0; e < E; ++e) o[e] = u; \
        break;                                            \
    }
        ECMD_FETCH_IN(0) ECMD_FETCH_IN(1) ECMD_FETCH_IN(2) ECMD_FETCH_IN(3)
        ECMD_FETCH_IN(4) ECMD_FETCH_IN(5) ECMD_FETCH_IN(6) ECMD_FETCH_IN(7)
        ECMD_FETCH_S(0) ECMD_FETCH_S(1) ECMD_FETCH_S(2) ECMD_FETCH_S(3)
        ECMD_FETCH_S(4) ECMD_FETCH_S(5) ECMD_FETCH_S(6) ECMD_FETCH_S(7)
        ECMD_FETCH_U(0) ECMD_FETCH_U(1) ECMD_FETCH_U(2) ECMD_FETCH_U(3)
        ECMD_FETCH_U(4) ECMD_FETCH_U(5) ECMD_FETCH_U(6) ECMD_FETCH_U(7)
#undef ECMD_FETCH_IN
#undef ECMD_FETCH_S
#undef ECMD_FETCH_U
    default:
        _Pragma("unroll") for (int e = 0; e < E; ++e) o[e] = 0u;
        break;
    }
}

template <int E>
__device__ __forceinline__ void rt_put(uint8_t dst, Regs<E> &R, const uint32_t (&v)[E])
{
    switch (dst) {
#define ECMD_PUT_S(k)                                     \
    case kRefSlot + k:                                    \
        _Pragma("unroll") for (int e = 0; e < E; ++e) R.s[k][e] = v[e]; \
        break;
        ECMD_PUT_S(0) ECMD_PUT_S(1) ECMD_PUT_S(2) ECMD_PUT_S(3)
        ECMD_PUT_S(4) ECMD_PUT_S(5) ECMD_PUT_S(6) ECMD_PUT_S(7)
#undef ECMD_PUT_S
    default:
        break;
    }
}

// Every opcode, for the interpreters' dispatch switches.
#define ECMD_FOR_EACH_CODE(X)                                                                  \
    X(C_MOV) X(C_ADD_F32) X(C_SUB_F32) X(C_MUL_F32) X(C_ADD_I32) X(C_SUB_I32) X(C_MUL_I32)      \
    X(C_NEG_F32) X(C_NEG_I32) X(C_NEG_F16) X(C_CVT_F16_F32) X(C_CVT_F32_F16) X(C_CVT_I32_F32)   \
    X(C_CVT_F32_I32) X(C_CVT_I32_F16) X(C_CVT_F16_I32)                                         \
    X(C_EQ_F32) X(C_NE_F32) X(C_LT_F32) X(C_LE_F32) X(C_GT_F32) X(C_GE_F32)                     \
    X(C_EQ_I32) X(C_NE_I32) X(C_LT_I32) X(C_LE_I32) X(C_GT_I32) X(C_GE_I32)                     \
    X(C_LT_U32) X(C_LE_U32) X(C_GT_U32) X(C_GE_U32)                                             \
    X(C_MIN_F32) X(C_MAX_F32) X(C_MIN_I32) X(C_MAX_I32) X(C_ABS_F32) X(C_ABS_I32) X(C_ABS_F16)  \
    X(C_SELECT) X(C_ADD_F16) X(C_SUB_F16) X(C_MUL_F16) X(C_ADD_BF16) X(C_SUB_BF16) X(C_MUL_BF16) \
    X(C_NEG_BF16) X(C_ABS_BF16) X(C_CVT_F16_BF16) X(C_CVT_BF16_F16) X(C_CVT_BF16_F32)           \
    X(C_CVT_F32_BF16) X(C_CVT_BF16_I32) X(C_CVT_I32_BF16)                                       \
    X(C_EQ_F16) X(C_NE_F16) X(C_LT_F16) X(C_LE_F16) X(C_GT_F16) X(C_GE_F16)                     \
    X(C_EQ_BF16) X(C_NE_BF16) X(C_LT_BF16) X(C_LE_BF16) X(C_GT_BF16) X(C_GE_BF16)               \
    X(C_MIN_F16) X(C_MAX_F16) X(C_MIN_BF16) X(C_MAX_BF16)
static_assert(C_COUNT == 70, "ECMD_FOR_EACH_CODE lists every opcode");

template <int E>
__device__ __forceinline__ void rt_apply(uint8_t code, const uint32_t (&a)[E], const uint32_t (&b)[E],
                                         const uint32_t (&c)[E], uint32_t (&r)[E])
{
    switch (code) {
#define ECMD_APPLY(k)                                     \
    case k:                                               \
        _Pragma("unroll") for (int e = 0; e < E; ++e) r[e] = apply<k>(a[e], b[e], c[e]); \
        break;
        ECMD_FOR_EACH_CODE(ECMD_APPLY)
#undef ECMD_APPLY
    default:
        _Pragma("unroll") for (int e = 0; e < E; ++e) r[e] = 0u;
        break;
    }
}

struct RtEval {
    static constexpr bool kSpecialised = false;
    __device__ static int n_in(const Program &P) { return P.n_in; }
    __device__ static int n_out(const Program &P) { return P.n_out; }
    __device__ static uint8_t in_ty(const Program &P, int k) { return P.in_ty[k]; }
    __device__ static uint8_t out_ty(const Program &P, int k) { return P.out_ty[k]; }

    template <int E>
    __device__ static __forceinline__ void run(const Program &P, const uint32_t *uni, Regs<E> &R,
                                               uint32_t (&out)[kMaxOut][E])
    {
        const int n_ops = P.n_ops;
        for (int i = 0; i < n_ops; ++i) {
            const TapeOp op = P.ops[i];
            uint32_t a[E], b[E], c[E], r[E];
            rt_fetch<E>(op.a, R, uni, a);
            rt_fetch<E>(op.b, R, uni, b);
            rt_fetch<E>(op.c, R, uni, c);
            rt_apply<E>(op.code, a, b, c, r);
            rt_put<E>(op.dst, R, r);
        }
#pragma unroll
        for (int k = 0; k < kMaxOut; ++k)
            if (k < P.n_out) rt_fetch<E>(P.out_ref[k], R, uni, out[k]);
    }
};

// ---------------------------------------------------------------------------
// Compile-time evaluator.

template <const Program &P>
struct CtEval {
    static constexpr bool kSpecialised = true;
    static constexpr const Program &kProg = P;
    __device__ static constexpr int n_in(const Program &) { return P.n_in; }
    __device__ static constexpr int n_out(const Program &) { return P.n_out; }
    __device__ static constexpr uint8_t in_ty(const Program &, int k) { return P.in_ty[k]; }
    __device__ static constexpr uint8_t out_ty(const Program &, int k) { return P.out_ty[k]; }

    template <uint8_t ref, int E>
    __device__ static __forceinline__ uint32_t get(const Regs<E> &R, const uint32_t *uni, int e)
    {
        if constexpr (ref == kRefNone) return 0u;
        else if constexpr (ref < kRefSlot) return R.in[ref - kRefIn][e];
        else if constexpr (ref < kRefUni) return R.s[ref - kRefSlot][e];
        else return uni[ref - kRefUni];
    }

    template <int I, int E>
    __device__ static __forceinline__ void step(const uint32_t *uni, Regs<E> &R)
    {
        if constexpr (I < P.n_ops) {
            constexpr TapeOp op = P.ops[I];
            uint32_t r[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                r[e] = apply<op.code>(get<op.a, E>(R, uni, e), get<op.b, E>(R, uni, e), get<op.c, E>(R, uni, e));
#pragma unroll
            for (int e = 0; e < E; ++e) R.s[op.dst - kRefSlot][e] = r[e];
            step<I + 1, E>(uni, R);
        }
    }

    template <int K, int E>
    __device__ static __forceinline__ void outs(const uint32_t *uni, const Regs<E> &R,
                                                uint32_t (&out)[kMaxOut][E])
    {
        if constexpr (K < P.n_out) {
#pragma unroll
            for (int e = 0; e < E; ++e) out[K][e] = get<P.out_ref[K], E>(R, uni, e);
            outs<K + 1, E>(uni, R, out);
        }
    }

    template <int E>
    __device__ static __forceinline__ void run(const Program &, const uint32_t *uni, Regs<E> &R,
                                               uint32_t (&out)[kMaxOut][E])
    {
        step<0, E>(uni, R);
        outs<0, E>(uni, R, out);
    }
};

// ---------------------------------------------------------------------------
// Global memory access for E consecutive elements of one operand.

template <int E, bool VEC>
__device__ __forceinline__ void load_elems(const void *p, uint8_t ty, int64_t i, int count,
                                           uint32_t (&v)[E])
{
    if (is16(ty)) {
        const uint16_t *q = static_cast<const uint16_t *>(p) + i;
        if constexpr (VEC) {
            static_assert(E % 8 == 0 || E == 4, "binary16 vectors are 8 or 4 wide");
            if constexpr (E % 8 == 0) {
#pragma unroll
                for (int w = 0; w < E / 8; ++w) {
                    const u32x4 d = reinterpret_cast<const u32x4 *>(q)[w];
                    const uint32_t x[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[8 * w + 2 * j] = x[j] & 0xffffu;
                        v[8 * w + 2 * j + 1] = x[j] >> 16;
                    }
                }
            } else {
                const u32x2 d = *reinterpret_cast<const u32x2 *>(q);
                v[0] = d.x & 0xffffu;
                v[1] = d.x >> 16;
                v[2] = d.y & 0xffffu;
                v[3] = d.y >> 16;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = e < count ? (uint32_t)q[e] : 0u;
        }
    } else {
        const uint32_t *q = static_cast<const uint32_t *>(p) + i;
        if constexpr (VEC) {
            static_assert(E % 4 == 0, "32-bit vectors are 4 wide");
#pragma unroll
            for (int w = 0; w < E / 4; ++w) {
                const u32x4 d = reinterpret_cast<const u32x4 *>(q)[w];
                v[4 * w + 0] = d.x;
                v[4 * w + 1] = d.y;
                v[4 * w + 2] = d.z;
                v[4 * w + 3] = d.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = e < count ? q[e] : 0u;
        }
    }
}

template <int E, bool VEC, bool NT>
__device__ __forceinline__ void store_elems(void *p, uint8_t ty, int64_t i, int count,
                                            const uint32_t (&v)[E])
{
    if (is16(ty)) {
        uint16_t *q = static_cast<uint16_t *>(p) + i;
        if constexpr (VEC) {
            if constexpr (E % 8 == 0) {
#pragma unroll
                for (int w = 0; w < E / 8; ++w) {
                    u32x4 d;
                    d.x = (v[8 * w + 0] & 0xffffu) | (v[8 * w + 1] << 16);
                    d.y = (v[8 * w + 2] & 0xffffu) | (v[8 * w + 3] << 16);
                    d.z = (v[8 * w + 4] & 0xffffu) | (v[8 * w + 5] << 16);
                    d.w = (v[8 * w + 6] & 0xffffu) | (v[8 * w + 7] << 16);
                    u32x4 *dst = reinterpret_cast<u32x4 *>(q) + w;
                    if constexpr (NT) __builtin_nontemporal_store(d, dst);
                    else *dst = d;
                }
            } else {
                u32x2 d;
                d.x = (v[0] & 0xffffu) | (v[1] << 16);
                d.y = (v[2] & 0xffffu) | (v[3] << 16);
                u32x2 *dst = reinterpret_cast<u32x2 *>(q);
                if constexpr (NT) __builtin_nontemporal_store(d, dst);
                else *dst = d;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e < count) q[e] = (uint16_t)v[e];
        }
    } else {
        uint32_t *q = static_cast<uint32_t *>(p) + i;
        if constexpr (VEC) {
#pragma unroll
            for (int w = 0; w < E / 4; ++w) {
                u32x4 d;
                d.x = v[4 * w + 0];
                d.y = v[4 * w + 1];
                d.z = v[4 * w + 2];
                d.w = v[4 * w + 3];
                u32x4 *dst = reinterpret_cast<u32x4 *>(q) + w;
                if constexpr (NT) __builtin_nontemporal_store(d, dst);
                else *dst = d;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e < count) q[e] = v[e];
        }
    }
}

// One vector access of G consecutive elements (G = 4 or 8) at element index i:
// 32-bit types move 16 bytes per 4 elements, binary16 8 bytes per 4.  With
// VEC false (unaligned views) the elements are accessed one by one, and only
// the first count of them.
template <bool NT, class T>
__device__ __forceinline__ T ld(const T *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// NTL: nontemporal loads ("nt" cache policy: the data is streamed, not kept).
template <int G, bool VEC, bool NTL = false>
__device__ __forceinline__ void load_group(const void *p, uint8_t ty, int64_t i, int count, uint32_t (&v)[G])
{
    static_assert(G == 4 || G == 8, "group of 4 or 8");
    if constexpr (VEC) {
        if (is16(ty)) {
            const uint16_t *q = static_cast<const uint16_t *>(p) + i;
            if constexpr (G == 8) {
                const u32x4 d = ld<NTL>(reinterpret_cast<const u32x4 *>(q));
                const uint32_t x[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = x[j] & 0xffffu;
                    v[2 * j + 1] = x[j] >> 16;
                }
            } else {
                const u32x2 d = ld<NTL>(reinterpret_cast<const u32x2 *>(q));
                v[0] = d.x & 0xffffu;
                v[1] = d.x >> 16;
                v[2] = d.y & 0xffffu;
                v[3] = d.y >> 16;
            }
        } else {
            const uint32_t *q = static_cast<const uint32_t *>(p) + i;
#pragma unroll
            for (int w = 0; w < G / 4; ++w) {
                const u32x4 d = ld<NTL>(reinterpret_cast<const u32x4 *>(q) + w);
                v[4 * w + 0] = d.x;
                v[4 * w + 1] = d.y;
                v[4 * w + 2] = d.z;
                v[4 * w + 3] = d.w;
            }
        }
    } else {
        load_elems<G, false>(p, ty, i, count, v);
    }
}

// load_group split in two, for code that picks between access forms at run
// time: load_raw issues the vector access of G elements at element index i
// and keeps the words as loaded (32-bit: G elements; 16-bit: G / 2 words of
// two elements), unpack_raw makes elements of them.  A use of a load's result
// inside the branch that issued it makes the wavefront wait for that load
// before it issues the next operand's; with the unpacking after every
// operand's loads, all of them are in flight together.
template <int G, bool NTL>
__device__ __forceinline__ void load_raw(const void *p, uint8_t ty, int64_t i, uint32_t (&raw)[G])
{
    static_assert(G == 4 || G == 8, "group of 4 or 8");
    if (is16(ty)) {
        const uint16_t *q = static_cast<const uint16_t *>(p) + i;
        if constexpr (G == 8) {
            const u32x4 d = ld<NTL>(reinterpret_cast<const u32x4 *>(q));
            raw[0] = d.x, raw[1] = d.y, raw[2] = d.z, raw[3] = d.w;
        } else {
            const u32x2 d = ld<NTL>(reinterpret_cast<const u32x2 *>(q));
            raw[0] = d.x, raw[1] = d.y;
        }
    } else {
        const uint32_t *q = static_cast<const uint32_t *>(p) + i;
#pragma unroll
        for (int w = 0; w < G / 4; ++w) {
            const u32x4 d = ld<NTL>(reinterpret_cast<const u32x4 *>(q) + w);
            raw[4 * w + 0] = d.x, raw[4 * w + 1] = d.y, raw[4 * w + 2] = d.z, raw[4 * w + 3] = d.w;
        }
    }
}

// The first count (< G) elements at element index i, one by one, laid out as
// load_raw lays out a whole vector (the rest zero).  Packing 16-bit elements
// waits for their loads, but only where some work-item takes this branch.
template <int G>
__device__ __forceinline__ void load_raw_elems(const void *p, uint8_t ty, int64_t i, int count, uint32_t (&raw)[G])
{
    if (is16(ty)) {
        const uint16_t *q = static_cast<const uint16_t *>(p) + i;
        uint32_t h[G];
#pragma unroll
        for (int e = 0; e < G; ++e) h[e] = e < count ? (uint32_t)q[e] : 0u;
#pragma unroll
        for (int w = 0; w < G / 2; ++w) raw[w] = h[2 * w] | (h[2 * w + 1] << 16);
    } else {
        const uint32_t *q = static_cast<const uint32_t *>(p) + i;
#pragma unroll
        for (int e = 0; e < G; ++e) raw[e] = e < count ? q[e] : 0u;
    }
}

template <int G>
__device__ __forceinline__ uint32_t unpack_raw(uint8_t ty, const uint32_t (&raw)[G], int e)
{
    if (is16(ty)) return (e & 1) ? raw[e >> 1] >> 16 : raw[e >> 1] & 0xffffu;
    return raw[e];
}

// Streaming stores of whole vectors through a buffer resource.  The
// nontemporal stores of store_group carry the `nt` bit only; with `sc1` as
// well (cache policy 18: nt sc1) a 1 GiB copy ran at 6,650 GB/s against
// 6,500, cold and back to back alike (same box, three runs, every word
// checked).  Global stores cannot carry sc1 from source, so these go through
// raw buffer stores, whose resource (base, size) must be uniform: `base` is
// a wavefront-uniform address, `off` the lane's byte offset from it, `bytes`
// the extent every lane's offset stays below (at most 2^32 - 1; stores past
// it would be dropped by the hardware's range check).
constexpr int kStreamPolicy = 18;             // nt sc1
constexpr int kBufferWord3 = 0x00020000;      // raw, untyped buffer resource for gfx950

__device__ __forceinline__ void *uniform_ptr(const void *p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
}

template <int G>
__device__ __forceinline__ void store_stream(void *base, uint32_t bytes, uint32_t off, uint8_t ty, const uint32_t (&v)[G])
{
    static_assert(G == 4 || G == 8, "group of 4 or 8");
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kBufferWord3);
    if (is16(ty)) {
        if constexpr (G == 8) {
            u32x4 d;
            d.x = (v[0] & 0xffffu) | (v[1] << 16);
            d.y = (v[2] & 0xffffu) | (v[3] << 16);
            d.z = (v[4] & 0xffffu) | (v[5] << 16);
            d.w = (v[6] & 0xffffu) | (v[7] << 16);
            __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, kStreamPolicy);
        } else {
            u32x2 d;
            d.x = (v[0] & 0xffffu) | (v[1] << 16);
            d.y = (v[2] & 0xffffu) | (v[3] << 16);
            __builtin_amdgcn_raw_buffer_store_b64(d, r, off, 0, kStreamPolicy);
        }
    } else {
#pragma unroll
        for (int w = 0; w < G / 4; ++w) {
            u32x4 d;
            d.x = v[4 * w + 0];
            d.y = v[4 * w + 1];
            d.z = v[4 * w + 2];
            d.w = v[4 * w + 3];
            __builtin_amdgcn_raw_buffer_store_b128(d, r, off + 16u * w, 0, kStreamPolicy);
        }
    }
}

template <int G, bool VEC, bool NT>
__device__ __forceinline__ void store_group(void *p, uint8_t ty, int64_t i, int count, const uint32_t (&v)[G])
{
    static_assert(G == 4 || G == 8, "group of 4 or 8");
    if constexpr (VEC) {
        if (is16(ty)) {
            uint16_t *q = static_cast<uint16_t *>(p) + i;
            if constexpr (G == 8) {
                u32x4 d;
                d.x = (v[0] & 0xffffu) | (v[1] << 16);
                d.y = (v[2] & 0xffffu) | (v[3] << 16);
                d.z = (v[4] & 0xffffu) | (v[5] << 16);
                d.w = (v[6] & 0xffffu) | (v[7] << 16);
                u32x4 *dst = reinterpret_cast<u32x4 *>(q);
                if constexpr (NT) __builtin_nontemporal_store(d, dst);
                else *dst = d;
            } else {
                u32x2 d;
                d.x = (v[0] & 0xffffu) | (v[1] << 16);
                d.y = (v[2] & 0xffffu) | (v[3] << 16);
                u32x2 *dst = reinterpret_cast<u32x2 *>(q);
                if constexpr (NT) __builtin_nontemporal_store(d, dst);
                else *dst = d;
            }
        } else {
            uint32_t *q = static_cast<uint32_t *>(p) + i;
#pragma unroll
            for (int w = 0; w < G / 4; ++w) {
                u32x4 d;
                d.x = v[4 * w + 0];
                d.y = v[4 * w + 1];
                d.z = v[4 * w + 2];
                d.w = v[4 * w + 3];
                u32x4 *dst = reinterpret_cast<u32x4 *>(q) + w;
                if constexpr (NT) __builtin_nontemporal_store(d, dst);
                else *dst = d;
            }
        }
    } else {
        store_elems<G, false, false>(p, ty, i, count, v);
    }
}

}  // namespace ecmd
