// quant.hip - block quantisers of weights, hidden states and the SwiGLU intermediate.
//
// NVFP4 with the 4-vs-6 block rule (AI Primer, "Thinking Machines releases Inkling 2
// Small weights under Apache 2.0", section "TL;DR") and MXFP8 (vLLM recipe
// "thinkingmachines/Inkling-2-Small", section "Overview"); activations are quantised
// to the layer's weight format (AI Primer, section "NVFP4 and MXFP8 experts").
// One thread owns one 16-block (NVFP4) or 32-block (MXFP8): the block is read with
// 16-byte loads, quantised in registers and written as packed bytes. Each NVFP4
// tensor scale needs the tensor's max |x| first, so NVFP4 runs as amax pass, block
// pass, then a tiny pass turning the amax into the fp32 tensor scale.
#include "act_quant.h"
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) fill_u32_kernel(uint32_t *p, uint32_t v, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// amax_bits[g] = max |x| over group g (x is `groups` consecutive groups of `per`
// bf16 values, `per` a multiple of 8). Max of non-negative floats equals the max
// of their bit patterns, so the cross-block step is an integer atomic max.
__global__ void __launch_bounds__(kThreads) amax_bf16_kernel(const uint16_t *__restrict__ x, int64_t per,
                                                             uint32_t *__restrict__ amax_bits) {
    const int g = blockIdx.y;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)g * per);
    const int64_t n8 = per / 8;
    uint32_t m = 0;  // max of |bf16| bit patterns (sign cleared); order-preserving
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = src[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m = max(m, w[j] & 0x7fffu);
            m = max(m, (w[j] >> 16) & 0x7fffu);
        }
    }
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
        if (m) atomic_max_grow(amax_bits + g, m << 16);  // bf16 bits -> fp32 bits
    }
}

// NVFP4 weights, in the packed tile layout (layout.h): thread b writes storage block
// b (codes at 8b, scale at b) from its source row and columns in the bf16 masters; the
// tensor scale comes from the expert's amax (fp32 bits, filled by amax_bf16_kernel).
__global__ void __launch_bounds__(kThreads) quant_w_nvfp4_kernel(const uint16_t *__restrict__ w, int64_t n_blocks,
                                                                 int64_t blocks_per_expert, int32_t K,
                                                                 const uint32_t *__restrict__ amax_bits,
                                                                 uint8_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ scales) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks; b += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = b / blocks_per_expert;
        int64_t n, k;
        layout::block_source(true, K, b - e * blocks_per_expert, n, k);
        const float sg = nvfp4_tensor_scale(__uint_as_float(amax_bits[e]));
        float x[16];
        load16_bf16(w + (e * (blocks_per_expert / (K / 16)) + n) * K + k, x);
        uint32_t lo, hi;
        int sc;
        nvfp4_quant_block(x, sg, lo, hi, sc);
        reinterpret_cast<uint2 *>(codes)[b] = make_uint2(lo, hi);
        scales[b] = (uint8_t)sc;
    }
}

__global__ void finish_tensor_scale_kernel(float *ts, int32_t n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) ts[i] = nvfp4_tensor_scale(ts[i]);
}

// MXFP8: one thread per 32-block. Hidden states (tile_K == 0): block b of a row-major
// [rows][K] bf16 tensor, codes row-major too; deq (optional) receives the exact bf16
// values code * 2^(scale - 127). Weights (tile_K == K): storage block b of the packed
// tile layout (layout.h), read from its source row and columns of [E][N][K] masters.
__global__ void __launch_bounds__(kThreads) quant_mxfp8_bf16_kernel(const uint16_t *__restrict__ x, int64_t n_blocks,
                                                                    int32_t tile_K, int64_t blocks_per_expert,
                                                                    uint8_t *__restrict__ codes,
                                                                    uint8_t *__restrict__ scales,
                                                                    uint16_t *__restrict__ deq) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks; b += (int64_t)gridDim.x * blockDim.x) {
        int64_t src_off = b * 32;
        if (tile_K) {
            const int64_t e = b / blocks_per_expert;
            int64_t n, k;
            layout::block_source(false, tile_K, b - e * blocks_per_expert, n, k);
            src_off = (e * (blocks_per_expert / (tile_K / 32)) + n) * tile_K + k;
        }
        const uint4 *src = reinterpret_cast<const uint4 *>(x + src_off);
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 u = src[q];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
        uint32_t c[8];
        const int sc = mxfp8_quant_block(v, c);
        uint4 *d0 = reinterpret_cast<uint4 *>(codes + b * 32), *d1 = d0 + 1;
        if (tile_K) {  // packed weights: the block's two 16-column quarters (layout.h)
            const int64_t e = b / blocks_per_expert;
            int64_t n, k;
            layout::block_source(false, tile_K, b - e * blocks_per_expert, n, k);
            uint8_t *ce = codes + e * blocks_per_expert * 32;
            d0 = reinterpret_cast<uint4 *>(ce + layout::code_offset(false, tile_K, n, k));
            d1 = reinterpret_cast<uint4 *>(ce + layout::code_offset(false, tile_K, n, k + 16));
        }
        *d0 = make_uint4(c[0], c[1], c[2], c[3]);
        *d1 = make_uint4(c[4], c[5], c[6], c[7]);
        scales[b] = (uint8_t)sc;
        if (deq) gemm_detail::store_dequant_mxfp8_32(deq + b * 32, c, sc);
    }
}

// MXFP4: one thread per 32-block. Hidden states (tile_K == 0): block b of a row-major
// [rows][K] bf16 tensor, codes [rows][K/2] row-major too. Weights (tile_K == K):
// storage block b of the packed MXFP4 tile layout (layout.h: 16 code bytes and one
// scale byte per 32-block, the two 32-column halves of a 32 x 64 tile apart), read from
// its source row and columns of [E][N][K] masters.
__global__ void __launch_bounds__(kThreads) quant_mxfp4_bf16_kernel(const uint16_t *__restrict__ x, int64_t n_blocks,
                                                                    int32_t tile_K, int64_t blocks_per_expert,
                                                                    uint8_t *__restrict__ codes,
                                                                    uint8_t *__restrict__ scales) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks; b += (int64_t)gridDim.x * blockDim.x) {
        int64_t src_off = b * 32;
        if (tile_K) {
            const int64_t e = b / blocks_per_expert;
            int64_t n, k;
            layout::block_source_mx4(tile_K, b - e * blocks_per_expert, n, k);
            src_off = (e * (blocks_per_expert / (tile_K / 32)) + n) * tile_K + k;
        }
        const uint4 *src = reinterpret_cast<const uint4 *>(x + src_off);
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 u = src[q];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
        uint32_t c[4];
        const int sc = mxfp4_quant_block(v, c);
        reinterpret_cast<uint4 *>(codes)[b] = make_uint4(c[0], c[1], c[2], c[3]);
        scales[b] = (uint8_t)sc;
    }
}

// FP8 weights (the fp8 variant of the vLLM recipe "thinkingmachines/Inkling-Small"): one
// wave per output channel (row n of expert e) of the bf16 masters [E][N][K]: the channel
// scale fl32(max |w| / 448) into channel_scales[e][n] and the E4M3 codes, each 16-column
// piece to its place in the MXFP8 tile layout (layout.h).
__global__ void __launch_bounds__(kThreads) quant_w_fp8_kernel(const uint16_t *__restrict__ w, int64_t n_rows,
                                                               int32_t N, int32_t K, uint8_t *__restrict__ codes,
                                                               float *__restrict__ channel_scales) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < n_rows; r += waves) {
        const int64_t e = r / N, n = r - e * N;
        uint8_t *ce = codes + e * N * (int64_t)K;
        const float s = fp8_row_quant(w + r * K, K, lane, [&](int i, uint4 c) {
            *reinterpret_cast<uint4 *>(ce + layout::code_offset(false, K, n, 16 * (int64_t)i)) = c;
        });
        if (lane == 0) channel_scales[r] = s;
    }
}

// FP8 SwiGLU intermediate: rows [0, S) of x [*][F] fp32, one wave per row: codes [S][F]
// row-major and the row scales [S].
__global__ void __launch_bounds__(kThreads) quant_inter_fp8_kernel(const float *__restrict__ x, int32_t F,
                                                                   const Ctrl *__restrict__ ctrl,
                                                                   uint8_t *__restrict__ codes,
                                                                   float *__restrict__ row_scales) {
    const int lane = threadIdx.x & 63;
    const int64_t n_rows = ctrl->S, waves = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < n_rows; r += waves) {
        uint8_t *dst = codes + r * F;
        const float s = fp8_row_quant(x + r * F, F, lane, [&](int i, uint4 c) { reinterpret_cast<uint4 *>(dst)[i] = c; });
        if (lane == 0) row_scales[r] = s;
    }
}

// Hidden states to the layer's format, one thread per block or one wave per FP8 row
// (act_quant.h).
__global__ void __launch_bounds__(kThreads) act_quant_kernel(const ActQuant q) {
    act_quant_range(q, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x);
}

// NVFP4 SwiGLU intermediate: rows [0, S) of x [*][F] fp32, one tensor scale over
// all S rows (max |x| gathered by the gate_up epilogue into ctrl->amax_i).
__global__ void __launch_bounds__(kThreads) quant_inter_nvfp4_kernel(const float *__restrict__ x, int32_t F,
                                                                     const Ctrl *__restrict__ ctrl,
                                                                     uint8_t *__restrict__ codes,
                                                                     uint8_t *__restrict__ scales,
                                                                     _Float16 *__restrict__ deq,
                                                                     float *__restrict__ tscale_out) {
    const float sg = nvfp4_tensor_scale(__uint_as_float(ctrl->amax_i));
    const int64_t n_blocks = (int64_t)ctrl->S * (F / 16);
    const int64_t b0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b0 == 0 && tscale_out) tscale_out[0] = sg;
    for (int64_t b = b0; b < n_blocks; b += (int64_t)gridDim.x * blockDim.x) {
        const float4 *src = reinterpret_cast<const float4 *>(x + b * 16);
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = src[q];
            v[4 * q] = f.x;
            v[4 * q + 1] = f.y;
            v[4 * q + 2] = f.z;
            v[4 * q + 3] = f.w;
        }
        uint32_t lo, hi;
        int sc;
        nvfp4_quant_block(v, sg, lo, hi, sc);
        reinterpret_cast<uint2 *>(codes)[b] = make_uint2(lo, hi);
        scales[b] = (uint8_t)sc;
        store_dequant16(deq + b * 16, lo, hi, sc);
    }
}

inline unsigned grid_for(int64_t n, int64_t cap = 1 << 20) {
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (unsigned)g;
}

}  // namespace

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n, 4096)), dim3(kThreads), 0, s, p, v, n);
    return hipGetLastError();
}

hipError_t launch_amax_bf16_rows(const uint16_t *x, int64_t rows, int64_t K, int64_t groups, uint32_t *amax_bits,
                                 hipStream_t s) {
    const int64_t per = rows * K / groups;
    int64_t bx = (per / 8 + kThreads * 8 - 1) / (kThreads * 8);  // about 8 loads per thread
    if (bx < 1) bx = 1;
    if (bx > 2048) bx = 2048;
    hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)bx, (unsigned)groups), dim3(kThreads), 0, s, x, per,
                       amax_bits);
    return hipGetLastError();
}

hipError_t launch_quant_weights_nvfp4(const uint16_t *w, int32_t E, int32_t N, int32_t K, const uint32_t *amax_bits,
                                      uint8_t *codes, uint8_t *scales, hipStream_t s) {
    const int64_t per = (int64_t)N * (K / 16);
    const int64_t nb = per * E;
    hipLaunchKernelGGL(quant_w_nvfp4_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, s, w, nb, per, K, amax_bits, codes,
                       scales);
    return hipGetLastError();
}

hipError_t launch_finish_tensor_scale(float *ts, int32_t n, hipStream_t s) {
    hipLaunchKernelGGL(finish_tensor_scale_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ts, n);
    return hipGetLastError();
}

hipError_t launch_quant_weights_mxfp8(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *codes,
                                      uint8_t *scales, hipStream_t s) {
    const int64_t per = (int64_t)N * (K / 32);
    const int64_t nb = per * E;
    hipLaunchKernelGGL(quant_mxfp8_bf16_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, s, w, nb, K, per, codes, scales,
                       (uint16_t *)nullptr);
    return hipGetLastError();
}

// Row-major pre-quantised weights (codes [E][N][K/2] NVFP4 and MXFP4, [E][N][K] MXFP8 and
// FP8; scales [E][N][K/16] or [E][N][K/32]) into the packed tile layout: one thread per
// quantisation block in storage order, the same mapping the quantisers write (layout.h).
// fmt: 1 NVFP4, 2 MXFP8, 3 MXFP4, 6 FP8 (the MOE_FMT_* values; FP8 has no block scales and
// moves its codes in MXFP8's 32-value pieces).
__global__ void __launch_bounds__(kThreads) pack_rowmajor_kernel(int fmt, const uint8_t *__restrict__ src_codes,
                                                                 const uint8_t *__restrict__ src_scales,
                                                                 int64_t n_blocks, int64_t blocks_per_expert,
                                                                 int32_t K, uint8_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ scales) {
    const int blk = fmt == 1 ? 16 : 32;                          // values per quantisation block
    const int64_t row_bytes = (fmt == 2 || fmt == 6) ? K : K / 2;  // code bytes per weight row
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks; b += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = b / blocks_per_expert, r = b - e * blocks_per_expert;
        int64_t n, k;
        if (fmt == 3)
            layout::block_source_mx4(K, r, n, k);
        else
            layout::block_source(fmt == 1, K, r, n, k);
        const int64_t row = e * (blocks_per_expert / (K / blk)) + n;  // weight row over all experts
        const uint8_t *src = src_codes + row * row_bytes + ((fmt == 2 || fmt == 6) ? k : k / 2);
        if (fmt == 1) {
            reinterpret_cast<uint2 *>(codes)[b] = *reinterpret_cast<const uint2 *>(src);
        } else if (fmt == 3) {
            reinterpret_cast<uint4 *>(codes)[b] = *reinterpret_cast<const uint4 *>(src);
        } else {
            uint8_t *ce = codes + e * blocks_per_expert * 32;
            *reinterpret_cast<uint4 *>(ce + layout::code_offset(false, K, n, k)) = *reinterpret_cast<const uint4 *>(src);
            *reinterpret_cast<uint4 *>(ce + layout::code_offset(false, K, n, k + 16)) =
                *reinterpret_cast<const uint4 *>(src + 16);
        }
        if (fmt != 6) scales[b] = src_scales[row * (K / blk) + k / blk];
    }
}

hipError_t launch_pack_rowmajor(int fmt, const uint8_t *src_codes, const uint8_t *src_scales, int32_t E, int32_t N,
                                int32_t K, uint8_t *codes, uint8_t *scales, hipStream_t s) {
    const int64_t per = (int64_t)N * (K / (fmt == 1 ? 16 : 32));
    const int64_t nb = per * E;
    hipLaunchKernelGGL(pack_rowmajor_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, s, fmt, src_codes, src_scales, nb,
                       per, K, codes, scales);
    return hipGetLastError();
}

// bf16 weights into the packed tile layout: one thread per 16-byte piece
__global__ void __launch_bounds__(kThreads) pack_bf16_kernel(const uint16_t *__restrict__ w, int64_t n_pieces,
                                                             int32_t K, int64_t pieces_per_expert,
                                                             uint8_t *__restrict__ codes) {
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n_pieces; r += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = r / pieces_per_expert;
        int64_t n, k;
        layout::piece_source_bf16(K, r - e * pieces_per_expert, n, k);
        const int64_t rows = pieces_per_expert / (K / 8);
        reinterpret_cast<uint4 *>(codes)[r] = *reinterpret_cast<const uint4 *>(w + (e * rows + n) * K + k);
    }
}

hipError_t launch_pack_weights_bf16(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *codes,
                                    hipStream_t s) {
    const int64_t per = (int64_t)N * (K / 8);
    const int64_t np = (int64_t)E * per;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(grid_for(np)), dim3(kThreads), 0, s, w, np, K, per, codes);
    return hipGetLastError();
}

hipError_t launch_quant_weights_mxfp4(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *codes,
                                      uint8_t *scales, hipStream_t s) {
    const int64_t per = (int64_t)N * (K / 32);
    const int64_t nb = (int64_t)E * per;
    hipLaunchKernelGGL(quant_mxfp4_bf16_kernel, dim3(grid_for(nb)), dim3(kThreads), 0, s, w, nb, K, per, codes,
                       scales);
    return hipGetLastError();
}




hipError_t launch_act_quant(const ActQuant &q, hipStream_t s) {
    const int64_t nb = act_quant_blocks(q);
    if (q.fmt == kActNone || nb == 0) return hipSuccess;
    hipLaunchKernelGGL(act_quant_kernel, dim3(grid_for(nb * act_quant_unit_threads(q))), dim3(kThreads), 0, s, q);
    return hipGetLastError();
}

hipError_t launch_quant_weights_fp8(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *codes,
                                    float *channel_scales, hipStream_t s) {
    const int64_t rows = (int64_t)E * N;
    hipLaunchKernelGGL(quant_w_fp8_kernel, dim3(grid_for(rows * 64)), dim3(kThreads), 0, s, w, rows, N, K, codes,
                       channel_scales);
    return hipGetLastError();
}

hipError_t launch_quant_inter_fp8(const float *x, int32_t max_rows, int32_t F, const Ctrl *ctrl, uint8_t *codes,
                                  float *row_scales, hipStream_t s) {
    hipLaunchKernelGGL(quant_inter_fp8_kernel, dim3(grid_for((int64_t)max_rows * 64, 4096)), dim3(kThreads), 0, s, x,
                       F, ctrl, codes, row_scales);
    return hipGetLastError();
}

hipError_t launch_quant_inter_nvfp4(const float *x, int32_t max_rows, int32_t F, const Ctrl *ctrl, uint8_t *codes,
                                    uint8_t *scales, _Float16 *deq, float *tscale_out, hipStream_t s) {
    const int64_t nb = (int64_t)max_rows * (F / 16);
    hipLaunchKernelGGL(quant_inter_nvfp4_kernel, dim3(grid_for(nb, 8192)), dim3(kThreads), 0, s, x, F, ctrl, codes,
                       scales, deq, tscale_out);
    return hipGetLastError();
}

}  // namespace moe
