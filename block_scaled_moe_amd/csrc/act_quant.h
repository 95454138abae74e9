// act_quant.h - per-block quantisation of the hidden states to the layer's format (AI
// Primer "Thinking Machines releases Inkling 2 Small weights under Apache 2.0", section
// "NVFP4 and MXFP8 experts": activations are quantised to the experts' format), shared by
// the standalone quantiser launch (quant.hip) and the permutation launch that carries it
// in extra workgroups (permute.hip). One call quantises one 16-value (NVFP4) or 32-value
// (MXFP8, MXFP4) block of the row-major [T][D] bf16 hidden states.
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

// number of quantisation blocks of the job
__host__ __device__ inline int64_t act_quant_blocks(const ActQuant &q) {
    return (int64_t)q.T * q.D / (q.fmt == kActNVFP4 ? 16 : 32);
}

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

}  // namespace moe
