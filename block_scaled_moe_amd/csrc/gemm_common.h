// gemm_common.h - exact 16-bit expansion of NVFP4 / MXFP8 codes for the gfx950 MFMAs,
// shared by the grouped GEMM kernels (tiled and streaming), for W4A4 / W8A8 layers and
// for NVFP4 weights with bf16 activations (W4A16).
//
// NVFP4 (E2M1 codes, E4M3 scale per 16; vLLM recipe "thinkingmachines/Inkling-2-Small",
// section "Overview"): c * s has at most 6 significant bits and lies in [2^-10, 2688],
// inside fp16's normal range, so v_cvt_scalef32_pk_f16_fp4 (whose scale operand only
// contributes an exponent, so it is given 1.0) followed by v_pk_mul_f16 by the E4M3
// scale forms each value exactly. MXFP8 (E4M3 codes, E8M0 scale per 32): E4M3 * 2^e has
// 4 significant bits; v_cvt_scalef32_pk_bf16_fp8 applies the E8M0 exponent exactly.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace gemm_detail {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// exact fp16 of a non-negative E4M3 scale byte (normal: rebias 7 -> 15; subnormal m*2^-9)
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c) {
    const uint32_t e = (c >> 3) & 15, m = c & 7;
    if (e == 0) return (_Float16)((float)m * 0x1p-9f);
    return __builtin_bit_cast(_Float16, (uint16_t)(((e + 8) << 10) | (m << 7)));
}

// 8 E2M1 codes (element i in nibble i) times the E4M3 scale s -> 8 exact fp16
__device__ __forceinline__ half8 dequant_nvfp4(uint32_t codes, _Float16 s) {
    const half2_t ss = {s, s};
    const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
    const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
    const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
    const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// 8 E2M1 codes (element i in nibble i) times the E4M3 scale value s -> 8 exact bf16
// (c * s has at most 6 significant bits). gfx950 has no packed bf16 multiply: two codes
// go to fp32 with the convert at scale 1, the two products are exact in fp32, and the
// pack to bf16 is exact.
__device__ __forceinline__ bf16x8 dequant_nvfp4_bf16(uint32_t codes, float s) {
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const float2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const float2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const float2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const float2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    bf16x8 r;
    r[0] = (__bf16)(c0[0] * s); r[1] = (__bf16)(c0[1] * s);
    r[2] = (__bf16)(c1[0] * s); r[3] = (__bf16)(c1[1] * s);
    r[4] = (__bf16)(c2[0] * s); r[5] = (__bf16)(c2[1] * s);
    r[6] = (__bf16)(c3[0] * s); r[7] = (__bf16)(c3[1] * s);
    return r;
}

// 8 E4M3 codes (element i in byte i) times 2^(e - 127) -> 8 exact bf16; `scale` is the
// float whose exponent field is the E8M0 byte e (the convert uses only the exponent).
__device__ __forceinline__ bf16x8 dequant_mxfp8(u32x2 codes, float scale) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, true);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// The 32 codes of one MXFP8 block (element i in byte i of cw) with E8M0 code sc, as 32
// exact bf16 values code * 2^(sc - 127) at dst (16-byte aligned). A block of scale code
// 0 (maximum below 2^-119) is expanded with the convert's own treatment of that scale.
__device__ __forceinline__ void store_dequant_mxfp8_32(void *dst, const uint32_t (&cw)[8], int sc) {
    const float scale = __uint_as_float((uint32_t)sc << 23);
    bf16x8 *d = reinterpret_cast<bf16x8 *>(dst);
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = dequant_mxfp8((u32x2){cw[2 * q], cw[2 * q + 1]}, scale);
}

// Work item w of a grouped GEMM's (M-tile, N-block) grid, expert-major: the items of one
// local expert are consecutive, and within it its M-tiles go in groups of up to G, each
// group sweeping every N-block (N-block outer, the group's tiles inner). Dealt to the
// XCDs in contiguous ranges, an expert's weight panel is fetched from HBM once per group
// and served to the group's other tiles by that XCD's L2, and a group's activation rows
// stay in L2 across its N-blocks. (Groups of G consecutive tiles regardless of expert
// re-fetched every panel a group straddling two experts touched: about twice the
// algorithmic weight traffic at prefill; one group per expert re-read a hot expert's
// activation rows once per N-block.) The tile list holds an expert's tiles
// consecutively, tile t starting at sorted row offsets[el] + (t - t0) bm, so the
// expert's first tile t0 and tile count te follow from any one of its tiles.
// Returns false for w past the n_tiles * NB items.
template <int G>
__device__ __forceinline__ bool expert_major_item(int w, int NB, int bm, int n_tiles, const int32_t *tile_expert,
                                                  const int32_t *tile_row0, const int32_t *offsets, int &tile,
                                                  int &nb) {
    if (w >= n_tiles * NB) return false;
    const int tq = w / NB;  // a tile of the expert that owns item w
    const int el = tile_expert[tq];
    const int o0 = offsets[el];
    const int t0 = tq - (tile_row0[tq] - o0) / bm;
    const int te = (offsets[el + 1] - o0 + bm - 1) / bm;
    const int local = w - NB * t0;             // < te * NB
    const int g = local / (G * NB), r = local % (G * NB);
    const int gs = min(G, te - g * G);         // tiles in group g (the last may be short)
    tile = t0 + g * G + r % gs;
    nb = r / gs;
    return true;
}

// SwiGLU g * u / (1 + exp(-g)) in fp32 from the hardware exp2 and reciprocal (about
// 1 ulp each). Rounding -g log2(e) adds about |g| 2^-24 relative error to exp(-g),
// which reaches the result weighted by exp(-g) / (1 + exp(-g)): the result is within
// a few ulps plus 1e-6 relative for |g| <= 16 and for every g > 0, and for g < -16 its
// error stays below 1e-11 |u|; once exp(-g) overflows the result is 0.
// y of the prefill-shaped down GEMMs: written once and read once by the combine, from
// HBM at these sizes, so stored non-temporally (skewed-mxfp8 down 1.92 -> 1.86 ms,
// prefill-fp8-ep4 0.372 -> 0.364 ms, prefill-nvfp4-ep4 unchanged)
__device__ __forceinline__ void store_y(float *p, float v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float swiglu(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace gemm_detail
}  // namespace moe
