// gemm_mx4.hip - grouped expert GEMMs for OCP MXFP4 experts (W4A4: E2M1 codes with an
// E8M0 scale per 32 values for both weights and activations; the AMD variant of the vLLM
// recipe "thinkingmachines/Inkling-Small", section "Variants") on the gfx950 scaled
// MFMA, v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands.
//
// The instruction takes the codes and E8M0 scales as they are stored: no expansion, no
// tensor scale. Lane l supplies row l % 32 of its operand over k = 32 (l / 32) .. +31 of
// the 64-wide K chunk, as 16 code bytes (element 2i in the low nibble) and the scale
// byte of that 32-block, which is exactly one half of a row's 32-byte slot in the packed
// weight layout (layout.h) and 16 contiguous bytes of a row-major activation row. Its
// products are exact and its fp32 accumulation measured no less accurate than a
// sequential fp32 sum (max error 1.6e-7 of the sum of |products| over K = 4096 with
// block exponents spread over +-12, 2.3e-8 at +-4, 0 with equal exponents).
//
//  - workgroup tile 64 sorted rows x 256 weight rows, 4 waves side by side in N, each
//    64 x 64 as 2 x 2 MFMA tiles; gate_up waves pair gate row f with up row F + f;
//  - every lane loads its A and B operands straight from global memory (the four waves
//    of a workgroup read the same activation rows, which the L1 serves), through a
//    register ring kMx4Ring chunks deep; no LDS and no barrier in the K loop;
//  - work items are grouped and dealt to the 8 XCDs as in the tile kernels;
//  - gate_up epilogue: SwiGLU in fp32, then each wave's 64 x 32 tile goes through LDS and
//    lane r quantises row r's 32-block to MXFP4 (16-byte code store, one scale byte).
// 32x32x64 operand layout (checked on gfx950 against an exact product): lane l holds row
// (or column) l % 32, k 32 (l / 32) .. +31; accumulator v of lane l is row 8(v/4) +
// 4(l/32) + v%4, column l%32.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

using namespace gemm_detail;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

#ifndef MOE_MX4_RING
#define MOE_MX4_RING 4
#endif
constexpr int kBM = 64, kMS = 2, kNS = 2, kBN = 128 * kNS, kThreads = 256, kGroup = 4;
constexpr int kMx4Ring = MOE_MX4_RING;
constexpr int kEpiStride = 33;  // floats per row of a wave's SwiGLU tile (bank spread)
constexpr int kCodeBlock = 32 * 32, kScaleBlock = 32 * 2;  // bytes per 32 x 64 weight block

__device__ __forceinline__ v8i fp4_operand(u32x4 c) {
    return (v8i){(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
}

template <bool GATE_UP>
__global__ void __launch_bounds__(kThreads, 2) mx4_gemm_kernel(const GemmArgs p) {
    __shared__ __attribute__((aligned(16))) float epi[GATE_UP ? 4 * kBM * kEpiStride : 4];

    const int K = p.K, N = p.N, F = N / 2;
    const int NB = GATE_UP ? F / (kBN / 2) : N / kBN;

    // ---- work item of this workgroup (XCD-contiguous ranges, as in the tile kernels)
    const int n_tiles = p.ctrl->n_tiles;
    const int total = (n_tiles + kGroup - 1) / kGroup * kGroup * NB;
    const int per_xcd = (total + 7) / 8;
    const int b = blockIdx.x;
    if ((b >> 3) >= per_xcd) return;
    const int w = (b & 7) * per_xcd + (b >> 3);
    if (w >= total) return;
    const int grp = w / (kGroup * NB), rem = w % (kGroup * NB);
    const int nb = rem / kGroup;
    const int tile = grp * kGroup + rem % kGroup;
    if (tile >= n_tiles) return;

    const int el = p.tile_expert[tile];
    const int p0 = p.tile_row0[tile];
    const int rows = min(kBM, p.offsets[el + 1] - p0);
    const int e = p.e_begin + el;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, g2 = lane >> 5;
    const int64_t kb = K / 64;  // 64-wide blocks per weight row group
    const uint8_t *wc_e = p.w_codes + (int64_t)e * N * (K / 2);
    const uint8_t *ws_e = p.w_scales + (int64_t)e * N * (K / 32);

    // ---- this lane's B operand rows (weights) and A operand rows (activations)
    const uint8_t *bc[kNS];
    const uint8_t *bs[kNS];
#pragma unroll
    for (int ns = 0; ns < kNS; ++ns) {
        int row;
        if (GATE_UP) {
            const int col = nb * (kBN / 2) + wave * 32 + l32;
            row = ns == 0 ? col : F + col;
        } else {
            row = nb * kBN + wave * 64 + 32 * ns + l32;
        }
        const int64_t blk0 = (int64_t)(row >> 5) * kb;
        bc[ns] = wc_e + blk0 * kCodeBlock + (row & 31) * 32 + 16 * g2;
        bs[ns] = ws_e + blk0 * kScaleBlock + (row & 31) * 2 + g2;
    }
    // rows past the tile's end read the tile's first row (in bounds; never stored)
    const uint8_t *ac[kMS];
    const uint8_t *as[kMS];
#pragma unroll
    for (int ms = 0; ms < kMS; ++ms) {
        const int r = 32 * ms + l32;
        const int pos = p0 + (r < rows ? r : 0);
        const int64_t arow = p.gather_by_token ? p.sorted_slot[pos] / p.top_k : pos;
        ac[ms] = p.a_codes + arow * (K / 2) + 16 * g2;
        as[ms] = p.a_scales + arow * (K / 32) + g2;
    }

    // ---- K loop: chunk c + kMx4Ring - 1 is loaded into ring slot (c - 1) % kMx4Ring while
    // chunk c is multiplied; loads past the end repeat the last chunk (in bounds, unused)
    u32x4 areg[kMx4Ring][kMS], breg[kMx4Ring][kNS];
    int asc[kMx4Ring][kMS], bsc[kMx4Ring][kNS];
    auto load = [&](int slot, int c) {
#pragma unroll
        for (int ms = 0; ms < kMS; ++ms) {
            areg[slot][ms] = *reinterpret_cast<const u32x4 *>(ac[ms] + 32 * (int64_t)c);
            asc[slot][ms] = as[ms][2 * c];
        }
#pragma unroll
        for (int ns = 0; ns < kNS; ++ns) {
            breg[slot][ns] = *reinterpret_cast<const u32x4 *>(bc[ns] + (int64_t)kCodeBlock * c);
            bsc[slot][ns] = bs[ns][(int64_t)kScaleBlock * c];
        }
    };
    float16_t acc[kMS][kNS];
#pragma unroll
    for (int i = 0; i < kMS; ++i)
#pragma unroll
        for (int j = 0; j < kNS; ++j) acc[i][j] = (float16_t){};
    const int n_chunks = K / 64;
#pragma unroll
    for (int r = 0; r < kMx4Ring - 1; ++r) load(r, min(r, n_chunks - 1));
    for (int c0 = 0; c0 < n_chunks; c0 += kMx4Ring) {
#pragma unroll
        for (int j = 0; j < kMx4Ring; ++j) {
            const int c = c0 + j;
            if (c >= n_chunks) break;
            load((j + kMx4Ring - 1) % kMx4Ring, min(c + kMx4Ring - 1, n_chunks - 1));
#pragma unroll
            for (int ms = 0; ms < kMS; ++ms)
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fp4_operand(areg[j][ms]), fp4_operand(breg[j][ns]), acc[ms][ns], 4, 4, 0, asc[j][ms], 0,
                        bsc[j][ns]);
        }
    }

    // ---- epilogue: accumulator v of lane l = row 32 ms + 8(v/4) + 4 g2 + v%4, column l32
    if (GATE_UP) {
        float *we = epi + wave * kBM * kEpiStride;
#pragma unroll
        for (int ms = 0; ms < kMS; ++ms)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                we[m * kEpiStride + l32] = swiglu(acc[ms][0][v], acc[ms][1][v]);
            }
        __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave complete in issue order
        const int m = lane;  // kBM == 64: one row per lane
        if (m < rows) {
            const int64_t row = p0 + m;
            const int fb = nb * (kBN / 2) + wave * 32;  // first column of this wave's block
            float x[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] = we[m * kEpiStride + i];
            uint32_t cw[4];
            const int sc = mxfp4_quant_block(x, cw);
            *reinterpret_cast<u32x4 *>(p.o_codes + row * (F / 2) + fb / 2) = (u32x4){cw[0], cw[1], cw[2], cw[3]};
            p.o_scales[row * (F / 32) + fb / 32] = (uint8_t)sc;
            if (p.o_tap) {
                float4 *t = reinterpret_cast<float4 *>(p.o_tap + row * F + fb);
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
            }
        }
    } else {
#pragma unroll
        for (int ms = 0; ms < kMS; ++ms)
#pragma unroll
            for (int ns = 0; ns < kNS; ++ns) {
                const int n = nb * kBN + wave * 64 + 32 * ns + l32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                    if (m < rows) p.out_f32[(int64_t)(p0 + m) * N + n] = acc[ms][ns][v];
                }
            }
    }
}

}  // namespace

static_assert(kBM == 64, "the MXFP4 kernels share the tile kernels' 64-row M-tiles");

bool mx4_gemm_supported(int32_t K, int32_t N, bool gate_up) {
    if (K <= 0 || N <= 0 || K % 64) return false;
    return gate_up ? (N % 2 == 0 && (N / 2) % (kBN / 2) == 0) : N % kBN == 0;
}

hipError_t launch_mx4_gemm(const GemmArgs &a, bool gate_up, int32_t max_tiles, hipStream_t s) {
    const int64_t nb = gate_up ? (a.N / 2) / (kBN / 2) : a.N / kBN;
    const int64_t items = (int64_t)(max_tiles + kGroup - 1) / kGroup * kGroup * nb;
    const int64_t grid = (items + 7) / 8 * 8;
    if (gate_up)
        hipLaunchKernelGGL((mx4_gemm_kernel<true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((mx4_gemm_kernel<false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
