// act_quant.h - per-block quantisation of the hidden states to the layer's format (AI
// Primer "Thinking Machines releases Inkling 2 Small weights under Apache 2.0", section
// "NVFP4 and MXFP8 experts": activations are quantised to the experts' format), shared by
// the standalone quantiser launch (quant.hip) and the permutation launch that carries it
// in extra workgroups (permute.hip). One call quantises one 16-value (NVFP4) or 32-value
// (MXFP8, MXFP4) block of the row-major [T][D] bf16 hidden states, or (FP8, one wave) one
// whole row.
#pragma once
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {

__device__ __forceinline__ void load16_bf16(const uint16_t *p, float (&x)[16]) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    const uint4 a = q[0], b = q[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}

__device__ __forceinline__ void load32_bf16(const uint16_t *p, float (&x)[32]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 u = src[q];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
            x[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
}

// exact fp16 of e2m1(code) * e4m3(scale) for the 16 codes of a block
__device__ __forceinline__ void store_dequant16(_Float16 *dst, uint32_t lo, uint32_t hi, int scale) {
    const _Float16 s = gemm_detail::e4m3_to_f16((uint32_t)scale);
    gemm_detail::half8 *d = reinterpret_cast<gemm_detail::half8 *>(dst);
    d[0] = gemm_detail::dequant_nvfp4(lo, s);
    d[1] = gemm_detail::dequant_nvfp4(hi, s);
}

__device__ __forceinline__ void load16_f32(const float *p, float (&x)[16]) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 v = q[j];
        x[4 * j] = v.x;
        x[4 * j + 1] = v.y;
        x[4 * j + 2] = v.z;
        x[4 * j + 3] = v.w;
    }
}
__device__ __forceinline__ void load16(const uint16_t *p, float (&x)[16]) { load16_bf16(p, x); }
__device__ __forceinline__ void load16(const float *p, float (&x)[16]) { load16_f32(p, x); }

// FP8 row (vLLM recipe "thinkingmachines/Inkling-Small", its fp8 variant: E4M3 with a
// dynamic scale per token; the scale fl32(max |x| / 448), 1 for an all-zero row, is the
// reading used for every row scale of the format): one wave quantises the K values of
// `row` (K % 16 == 0), lane l taking 16-value pieces l, l + 64, ...; first the row
// maximum, then the codes E4M3(fl32(x / s)) (nearest even, saturating), piece i handed to
// store(i, codes) as 16 bytes. Returns s (every lane).
template <typename Src, typename Store>
__device__ __forceinline__ float fp8_row_quant(const Src *row, int K, int lane, Store store) {
    const int n_pieces = K / 16;
    float amax = 0.0f;
    for (int i = lane; i < n_pieces; i += 64) {
        float x[16];
        load16(row + 16 * i, x);
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(x[j]));
    }
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int i = lane; i < n_pieces; i += 64) {
        float x[16];
        load16(row + 16 * i, x);
        uint32_t c[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float v0 = e4m3_clamp(x[4 * w] / s), v1 = e4m3_clamp(x[4 * w + 1] / s);
            const float v2 = e4m3_clamp(x[4 * w + 2] / s), v3 = e4m3_clamp(x[4 * w + 3] / s);
            c[w] = e4m3_pack2<true>(e4m3_pack2<false>(0u, v0, v1), v2, v3);
        }
        store(i, make_uint4(c[0], c[1], c[2], c[3]));
    }
    return s;
}

// FP8 hidden-state row t: codes [T][D] row-major and the row scale
__device__ __forceinline__ void act_quant_fp8_row(const ActQuant &q, int64_t t, int lane) {
    uint8_t *dst = q.codes + t * q.D;
    const float s = fp8_row_quant(q.h + t * q.D, q.D, lane,
                                  [&](int i, uint4 c) { reinterpret_cast<uint4 *>(dst)[i] = c; });
    if (lane == 0) q.row_scales[t] = s;
}

// number of work units of the job: quantisation blocks (one thread each) or, for FP8,
// rows (one wave each)
__host__ __device__ inline int64_t act_quant_blocks(const ActQuant &q) {
    if (q.fmt == kActFP8) return q.T;
    return (int64_t)q.T * q.D / (q.fmt == kActNVFP4 ? 16 : 32);
}
__host__ __device__ inline int act_quant_unit_threads(const ActQuant &q) { return q.fmt == kActFP8 ? 64 : 1; }

// Units [first, first + stride, ...) of the job for the thread `tid` of `n_threads`
// (a multiple of 64) working on it.
__device__ __forceinline__ void act_quant_range(const ActQuant &q, int64_t tid, int64_t n_threads);

// Block b of the job: NVFP4 (one tensor scale over all of h, from amax_bits; codes,
// E4M3 scales, the exact fp16 values and, from block 0, the tensor scale), MXFP8 (codes,
// E8M0 scales and, if deq is set, the exact bf16 values) or MXFP4 (codes, E8M0 scales).
__device__ __forceinline__ void act_quant_block(const ActQuant &q, int64_t b) {
    if (q.fmt == kActNVFP4) {
        const float sg = nvfp4_tensor_scale(__uint_as_float(q.amax_bits[0]));
        if (b == 0 && q.tscale_out) q.tscale_out[0] = sg;
        float x[16];
        load16_bf16(q.h + b * 16, x);
        uint32_t lo, hi;
        int sc;
        nvfp4_quant_block(x, sg, lo, hi, sc);
        reinterpret_cast<uint2 *>(q.codes)[b] = make_uint2(lo, hi);
        q.scales[b] = (uint8_t)sc;
        store_dequant16(static_cast<_Float16 *>(q.deq) + b * 16, lo, hi, sc);
    } else if (q.fmt == kActMXFP8) {
        float x[32];
        load32_bf16(q.h + b * 32, x);
        uint32_t c[8];
        const int sc = mxfp8_quant_block(x, c);
        uint4 *d = reinterpret_cast<uint4 *>(q.codes + b * 32);
        d[0] = make_uint4(c[0], c[1], c[2], c[3]);
        d[1] = make_uint4(c[4], c[5], c[6], c[7]);
        q.scales[b] = (uint8_t)sc;
        if (q.deq) gemm_detail::store_dequant_mxfp8_32(static_cast<uint16_t *>(q.deq) + b * 32, c, sc);
    } else {
        float x[32];
        load32_bf16(q.h + b * 32, x);
        uint32_t c[4];
        const int sc = mxfp4_quant_block(x, c);
        reinterpret_cast<uint4 *>(q.codes)[b] = make_uint4(c[0], c[1], c[2], c[3]);
        q.scales[b] = (uint8_t)sc;
    }
}

__device__ __forceinline__ void act_quant_range(const ActQuant &q, int64_t tid, int64_t n_threads) {
    const int64_t n = act_quant_blocks(q);
    if (q.fmt == kActFP8) {
        const int lane = (int)(tid & 63);
        for (int64_t r = tid >> 6; r < n; r += n_threads >> 6) act_quant_fp8_row(q, r, lane);
    } else {
        for (int64_t b = tid; b < n; b += n_threads) act_quant_block(q, b);
    }
}

}  // namespace moe
