// formats.h - device-side element and scale formats of the block-scaled experts.
//
// NVFP4 (E2M1 codes, E4M3 scale per 16, fp32 tensor scale) with the 4-vs-6 block
// rule of AI Primer, "Thinking Machines releases Inkling 2 Small weights under
// Apache 2.0", section "TL;DR"; MXFP8 (E4M3 codes, E8M0 scale per 32) named in
// the vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview"; MXFP4
// (E2M1 codes, E8M0 scale per 32) as in the AMD variant of the vLLM recipe
// "thinkingmachines/Inkling-Small", section "Variants".
//
// Every floating-point step below is one IEEE binary32 operation with
// round-to-nearest-even: the library is compiled with -ffp-contract=off,
// correctly rounded fp32 division and fp32 denormals kept, so that the codes and
// scales are a deterministic function of the input values.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- E2M1
// Value of a 4-bit E2M1 code: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0.
__device__ __forceinline__ float e2m1_value(int c) {
    const int mag = c & 7;
    float v;
    if (mag < 2) {
        v = 0.5f * (float)mag;
    } else {
        v = __uint_as_float(((uint32_t)((mag >> 1) + 126) << 23) | ((uint32_t)(mag & 1) << 22));
    }
    return (c & 8) ? -v : v;
}

// Nearest E2M1 code to y, ties to the even code, saturating at 6; the sign of y
// (including -0) is kept. Magnitudes: 0, .5, 1, 1.5, 2, 3, 4, 6; the decision
// points are the midpoints, each tie going to the code with mantissa bit 0.
__device__ __forceinline__ int e2m1_encode(float y) {
    const float a = fabsf(y);
    const int c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                  (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(y) >> 28) & 8);
}

// ---------------------------------------------------------------- E4M3 (OCP "FN")
// Value of a non-negative E4M3 code 0x00..0x7E (bias 7; subnormals m * 2^-9).
__device__ __forceinline__ float e4m3_value_pos(int c) {
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 0) return (float)m * 0x1p-9f;
    return __uint_as_float(((uint32_t)(e + 120) << 23) | ((uint32_t)m << 20));
}

// Nearest E4M3 code to a >= 0, ties to even, saturating at 448 (0x7E; never NaN).
// Normal range: spacing 2^(E-3) for a in [2^E, 2^(E+1)), E >= -6; below 2^-6 the
// spacing is 2^-9 (subnormals). Scaling by a power of two is exact, and rintf
// rounds half to even, so the code index parity follows the mantissa parity.
__device__ __forceinline__ int e4m3_encode_pos(float a) {
    if (!(a < 448.0f)) return 0x7E;
    const int E = (int)(__float_as_uint(a) >> 23) - 127;
    if (E < -6) return (int)rintf(a * 512.0f);
    const float n = rintf(ldexpf(a, 3 - E));  // in [8, 16]
    return ((E + 7) << 3) + (int)n - 8;
}

__device__ __forceinline__ int e4m3_encode(float v) {
    return e4m3_encode_pos(fabsf(v)) | ((__float_as_uint(v) >> 24) & 0x80);
}

// ---------------------------------------------------------------- E8M0
// MXFP8 block scale code for a block maximum: the exponent floor(log2 amax) - 8
// taken from the fp32 exponent field, clamped to [-127, 127], plus bias 127;
// amax == 0 gives code 0.
__device__ __forceinline__ int e8m0_code_for_amax(float amax) {
    if (!(amax > 0.0f)) return 0;
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    int se = ef - 127 - 8;  // a subnormal amax (ef == 0) lands below -127 as well
    if (se < -127) se = -127;
    return se + 127;
}

// ---------------------------------------------------------------- NVFP4 tensor scale
__device__ __forceinline__ float nvfp4_tensor_scale(float amax) {
    return amax > 0.0f ? amax / 2688.0f : 1.0f;  // 2688 = 6 * 448
}

// ---------------------------------------------------------------- NVFP4 block
// E2M1 codes of two values into byte SEL of `old` (element a in the low nibble). The
// gfx950 convert rounds to nearest even, saturates at 6 and keeps the sign of -0; with
// scale 1.0 it equals e2m1_encode for every finite fp32 input (checked exhaustively on
// the device). Its scale operand only contributes an exponent, so 1.0 is passed.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// The two E2M1 values of byte SEL of `codes`, exact.
template <int SEL>
__device__ __forceinline__ void e2m1_unpack2(uint32_t codes, float &a, float &b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
    a = v.x;
    b = v.y;
}

// fl(x / S) for 2^-100 <= S <= 2^100 and |x / S| in [2^-3, 2^8], one multiply and two
// fused multiply-adds instead of a division: with R = fl(1 / S) and q0 = fl(|x| R),
// the remainder |x| - q0 S is exact and fl(q0 + (|x| - q0 S) R) is the correctly
// rounded quotient (Markstein's theorem; P. Markstein, IBM J. Res. Dev. 34(1), 1990).
// Outside that quotient range the result is still within a few ulps of the quotient,
// which is enough for the E2M1 encoding: below 2^-3 every such value encodes to a
// signed zero, above 2^8 to the saturated code. The sign is taken from x, so -0 stays.
__device__ __forceinline__ float quotient_by(float x, float S, float R) {
    const float ax = fabsf(x);
    const float q0 = ax * R;
    return copysignf(fmaf(fmaf(-q0, S, ax), R, q0), x);
}

// One candidate of the 4-vs-6 rule: the block maximum r (already divided by the
// tensor scale sg) is mapped to M; returns the fp32 sum of squared errors (in
// element order) and the codes (nibbles packed, element 2i in the low nibble).
// Element i's code is the E2M1 encoding of fl(x[i] / S), S = fl(e4m3(r / M) * sg).
__device__ __forceinline__ float nvfp4_candidate(const float (&x)[16], float r, float sg, float M,
                                                 uint32_t &lo, uint32_t &hi, int &scode) {
    const float t = r / M;
    scode = e4m3_encode_pos(t);
    const float sdec = e4m3_value_pos(scode);
    const float S = sdec * sg;
    float err = 0.0f;
    if (S >= 0x1p-100f && S <= 0x1p100f) {
        const float R = 1.0f / S;
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = quotient_by(x[i], S, R);
        lo = e2m1_pack2<0>(0u, q[0], q[1]);
        lo = e2m1_pack2<1>(lo, q[2], q[3]);
        lo = e2m1_pack2<2>(lo, q[4], q[5]);
        lo = e2m1_pack2<3>(lo, q[6], q[7]);
        hi = e2m1_pack2<0>(0u, q[8], q[9]);
        hi = e2m1_pack2<1>(hi, q[10], q[11]);
        hi = e2m1_pack2<2>(hi, q[12], q[13]);
        hi = e2m1_pack2<3>(hi, q[14], q[15]);
        float v[16];
        e2m1_unpack2<0>(lo, v[0], v[1]);
        e2m1_unpack2<1>(lo, v[2], v[3]);
        e2m1_unpack2<2>(lo, v[4], v[5]);
        e2m1_unpack2<3>(lo, v[6], v[7]);
        e2m1_unpack2<0>(hi, v[8], v[9]);
        e2m1_unpack2<1>(hi, v[10], v[11]);
        e2m1_unpack2<2>(hi, v[12], v[13]);
        e2m1_unpack2<3>(hi, v[14], v[15]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = x[i] - v[i] * S;
            err = err + e * e;
        }
        return err;
    }
    // scales at the ends of the fp32 range (including S == 0): one division per element
    lo = 0;
    hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int c;
        if (sdec == 0.0f) {
            c = (__float_as_uint(x[i]) >> 28) & 8;
        } else {
            c = e2m1_encode(x[i] / S);
        }
        const float deq = e2m1_value(c) * S;
        const float e = x[i] - deq;
        err = err + e * e;
        if (i < 8) lo |= (uint32_t)c << (4 * i);
        else hi |= (uint32_t)c << (4 * (i - 8));
    }
    return err;
}

// Quantise one 16-block with tensor scale sg: 8 code bytes (lo, hi words) and one
// E4M3 scale byte; keeps the max->4 candidate only when its error is strictly lower.
__device__ __forceinline__ void nvfp4_quant_block(const float (&x)[16], float sg, uint32_t &lo,
                                                  uint32_t &hi, int &scale) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const float r = amax / sg;
    uint32_t lo6, hi6, lo4, hi4;
    int s6, s4;
    const float err6 = nvfp4_candidate(x, r, sg, 6.0f, lo6, hi6, s6);
    const float err4 = nvfp4_candidate(x, r, sg, 4.0f, lo4, hi4, s4);
    const bool take4 = err4 < err6;
    lo = take4 ? lo4 : lo6;
    hi = take4 ? hi4 : hi6;
    scale = take4 ? s4 : s6;
}

// ---------------------------------------------------------------- MXFP8 block
// E4M3 codes of two values into the low (HI false) or high 16 bits of `old` (a in the
// lower byte). The gfx950 convert rounds to nearest even and equals e4m3_encode for
// every fp32 input of magnitude <= 448 (checked exhaustively on the device); it does
// not saturate above that, so callers clamp first (e4m3_clamp).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(uint32_t old, float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// v clamped to [-448, 448]: the E4M3 code of the result is e4m3_encode(v)
__device__ __forceinline__ float e4m3_clamp(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// Quantise one 32-block: E8M0 scale code and 32 E4M3 codes of x * 2^-exponent
// (a power-of-two scaling, exact for every value whose code is not zero).
__device__ __forceinline__ int mxfp8_quant_block(const float (&x)[32], uint32_t (&codes)[8]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const int sc = e8m0_code_for_amax(amax);
    const int se = sc - 127;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const float v0 = e4m3_clamp(ldexpf(x[4 * w], -se)), v1 = e4m3_clamp(ldexpf(x[4 * w + 1], -se));
        const float v2 = e4m3_clamp(ldexpf(x[4 * w + 2], -se)), v3 = e4m3_clamp(ldexpf(x[4 * w + 3], -se));
        codes[w] = e4m3_pack2<true>(e4m3_pack2<false>(0u, v0, v1), v2, v3);
    }
    return sc;
}

// ---------------------------------------------------------------- MXFP4 block
// OCP MXFP4 (vLLM recipe "thinkingmachines/Inkling-Small", section "Variants": the AMD
// checkpoint's W4A4 experts): E2M1 codes with one E8M0 scale per 32 values,
// 2^(floor(log2 amax) - 2) (E2M1's largest exponent is 2), exponent clamped to
// [-127, 127], code 0 when amax == 0.
__device__ __forceinline__ int mxfp4_scale_code(float amax) {
    if (!(amax > 0.0f)) return 0;
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    int se = ef - 127 - 2;  // a subnormal amax (ef == 0) lands below -127 as well
    if (se < -127) se = -127;
    return se + 127;
}

// Quantise one 32-block: E8M0 scale code and 32 E2M1 codes of x * 2^-exponent packed
// two per byte (element 2i in the low nibble); the power-of-two scaling is exact for
// every value whose code is not zero, and the convert saturates at 6.
__device__ __forceinline__ int mxfp4_quant_block(const float (&x)[32], uint32_t (&codes)[4]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const int sc = mxfp4_scale_code(amax);
    const int se = sc - 127;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t v = e2m1_pack2<0>(0u, ldexpf(x[8 * w], -se), ldexpf(x[8 * w + 1], -se));
        v = e2m1_pack2<1>(v, ldexpf(x[8 * w + 2], -se), ldexpf(x[8 * w + 3], -se));
        v = e2m1_pack2<2>(v, ldexpf(x[8 * w + 4], -se), ldexpf(x[8 * w + 5], -se));
        codes[w] = e2m1_pack2<3>(v, ldexpf(x[8 * w + 6], -se), ldexpf(x[8 * w + 7], -se));
    }
    return sc;
}

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// *p = max(*p, v) for fp32 bit patterns of non-negative values (integer order). The
// stored value only grows, so a v that does not exceed what is already there changes
// nothing and skips the atomic: most callers of one accumulator then only read it.
__device__ __forceinline__ void atomic_max_grow(uint32_t *p, uint32_t v) {
    if (v > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, v);
}

}  // namespace moe
