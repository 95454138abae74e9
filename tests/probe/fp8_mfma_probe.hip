// fp8_mfma_probe.hip - accuracy characterisation of the gfx950 MFMA routes for MXFP8
// dot products (OCP MX: E4M3 codes with one E8M0 scale per 32 values). Test
// infrastructure only: tests/test_gpu_fp8_mfma_accuracy.py loads it and compares the
// results with exact dot products formed on the host.
//
// One wave computes one 32 x 32 tile C[m][n] = sum_k A[m][k] B[n][k] over K (a multiple
// of 64), with A and B stored row-major as codes [32][K] and scales [32][K/32].
//  mode 0: v_mfma_scale_f32_32x32x64_f8f6f4 on the codes and scales as stored; `group`
//          consecutive 64-wide K chunks are chained through the MFMA accumulator, then
//          that partial is added to an fp32 sum with an ordinary (round-to-nearest) add
//          and the MFMA accumulator restarts from zero. group = K / 64 chains all of K.
//          `layout` picks which k of the chunk lane half g = l / 32 places in its eight
//          operand registers (the same for A and B, so the sum is unchanged up to order;
//          only the block each k is scaled by depends on it). Registers 0-3 hold bytes
//          0-15 and registers 4-7 bytes 16-31 of the lane's operand:
//            0: k = 32 g .. 32 g + 31
//            1: k = 16 g .. +15, then 32 + 16 g .. +15
//            2: k = 16 i + 8 g .. +7 for i = 0..3 (four 8-byte pieces)
//          The scale operand of lane l is the E8M0 byte of row l % 32 and block l / 32.
//  mode 1: each code expanded exactly to bf16 with its block scale applied
//          (v_cvt_scalef32_pk_bf16_fp8), then v_mfma_f32_32x32x16_bf16 chained over K.
// Operand layouts: 32x32x64 - lane l supplies row (column) l % 32 (k as above);
// 32x32x16 - lane l supplies
// row (column) l % 32, k 8 (l / 32) .. +7 of the step. Accumulator v of lane l is row
// 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32 for both shapes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 expand8(u32x2 c, float scale) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, scale, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, scale, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, scale, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, scale, true);
    return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// the lane's 32 operand bytes of one 64-wide chunk starting at p (16-byte aligned)
__device__ __forceinline__ v8i operand(const uint8_t *p, int layout, int g) {
    u32x4 lo, hi;
    if (layout == 0) {
        lo = *reinterpret_cast<const u32x4 *>(p + 32 * g);
        hi = *reinterpret_cast<const u32x4 *>(p + 32 * g + 16);
    } else if (layout == 1) {
        lo = *reinterpret_cast<const u32x4 *>(p + 16 * g);
        hi = *reinterpret_cast<const u32x4 *>(p + 32 + 16 * g);
    } else {
        const u32x2 q0 = *reinterpret_cast<const u32x2 *>(p + 8 * g);
        const u32x2 q1 = *reinterpret_cast<const u32x2 *>(p + 16 + 8 * g);
        const u32x2 q2 = *reinterpret_cast<const u32x2 *>(p + 32 + 8 * g);
        const u32x2 q3 = *reinterpret_cast<const u32x2 *>(p + 48 + 8 * g);
        lo = (u32x4){q0.x, q0.y, q1.x, q1.y};
        hi = (u32x4){q2.x, q2.y, q3.x, q3.y};
    }
    return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__global__ void __launch_bounds__(64) probe_kernel(int mode, int group, int layout, int K, const uint8_t *a,
                                                   const uint8_t *as,
                                                   const uint8_t *b, const uint8_t *bs, float *out) {
    const int tile = blockIdx.x, l = threadIdx.x, r = l & 31, g = l >> 5;
    const uint8_t *ar = a + ((int64_t)tile * 32 + r) * K;
    const uint8_t *br = b + ((int64_t)tile * 32 + r) * K;
    const uint8_t *asr = as + ((int64_t)tile * 32 + r) * (K / 32);
    const uint8_t *bsr = bs + ((int64_t)tile * 32 + r) * (K / 32);
    v16f sum = {};
    if (mode == 0) {
        v16f acc = {};
        const int n_chunks = K / 64;
        for (int c = 0; c < n_chunks; ++c) {
            const v8i va = operand(ar + 64 * c, layout, g), vb = operand(br + 64 * c, layout, g);
            const int sa = asr[2 * c + g], sb = bsr[2 * c + g];
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 0, 0, 0, sa, 0, sb);
            if ((c + 1) % group == 0 || c + 1 == n_chunks) {
#pragma unroll
                for (int v = 0; v < 16; ++v) sum[v] = sum[v] + acc[v];
                acc = (v16f){};
            }
        }
    } else {
        for (int k0 = 0; k0 < K; k0 += 16) {
            const int k = k0 + 8 * g;
            const u32x2 ca = *reinterpret_cast<const u32x2 *>(ar + k);
            const u32x2 cb = *reinterpret_cast<const u32x2 *>(br + k);
            const float fa = __uint_as_float((uint32_t)asr[k / 32] << 23);
            const float fb = __uint_as_float((uint32_t)bsr[k / 32] << 23);
            sum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(expand8(ca, fa), expand8(cb, fb), sum, 0, 0, 0);
        }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v / 4) + 4 * g + (v % 4);
        out[((int64_t)tile * 32 + m) * 32 + r] = sum[v];
    }
}

}  // namespace

// Device pointers; a, b: [tiles][32][K] E4M3 codes; as, bs: [tiles][32][K / 32] E8M0
// codes (every scale code must be at least 1: the convert of mode 1 reads a scale code
// of 0 as the float 0); out: [tiles][32][32] fp32. Returns 0, -1 for invalid arguments
// (nothing launched) or -5 if the launch failed. Runs on the default stream.
extern "C" int fp8_probe(int mode, int group, int layout, int K, int tiles, const uint8_t *a, const uint8_t *as,
                         const uint8_t *b, const uint8_t *bs, float *out) {
    if ((mode != 0 && mode != 1) || group < 1 || layout < 0 || layout > 2 || K <= 0 || K % 64 || tiles <= 0)
        return -1;
    if (!a || !as || !b || !bs || !out) return -1;
    if (((uintptr_t)a | (uintptr_t)b) & 15) return -1;
    hipLaunchKernelGGL(probe_kernel, dim3(tiles), dim3(64), 0, 0, mode, group, layout, K, a, as, b, bs, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
