// formats.h - device-side element and scale formats of the block-scaled experts.
//
// NVFP4 (E2M1 codes, E4M3 scale per 16, fp32 tensor scale) with the 4-vs-6 block
// rule of AI Primer, "Thinking Machines releases Inkling 2 Small weights under
// Apache 2.0", section "TL;DR"; MXFP8 (E4M3 codes, E8M0 scale per 32) named in
// the vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview".
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
// One candidate of the 4-vs-6 rule: the block maximum r (already divided by the
// tensor scale sg) is mapped to M; returns the fp32 sum of squared errors (in
// element order) and the codes (nibbles packed, element 2i in the low nibble).
__device__ __forceinline__ float nvfp4_candidate(const float (&x)[16], float r, float sg, float M,
                                                 uint32_t &lo, uint32_t &hi, int &scode) {
    const float t = r / M;
    scode = e4m3_encode_pos(t);
    const float sdec = e4m3_value_pos(scode);
    const float S = sdec * sg;
    float err = 0.0f;
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
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= (uint32_t)e4m3_encode(ldexpf(x[4 * w + b], -se)) << (8 * b);
        codes[w] = v;
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
