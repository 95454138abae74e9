// gemm.hip - grouped expert GEMMs (gate_up with the SwiGLU epilogue, and down) for
// NVFP4 and MXFP8 expert layers on gfx950 MFMA.
//
// Expert formats (vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview";
// AI Primer "Thinking Machines releases Inkling 2 Small weights under Apache 2.0",
// section "NVFP4 and MXFP8 experts"): NVFP4 = E2M1 codes, an E4M3 scale per 16 and an
// fp32 tensor scale; MXFP8 = E4M3 codes and an E8M0 scale per 32. Activations arrive
// in the same format, already expanded to their exact 16-bit values; or, for NVFP4
// weights with bf16 activations (W4A16, vLLM recipe "thinkingmachines/Inkling-Small",
// section "Variants"), as the bf16 values themselves, with the weights expanded to bf16.
//
// Arithmetic: every weight value is formed EXACTLY in a 16-bit float and fed to a
// 16x16x32 MFMA with fp32 accumulation, so all products are exact and the sums are
// ordinary fp32 accumulations.
//  - NVFP4: c * s has at most 6 significant bits and lies in [2^-10, 2688], inside
//    fp16's normal range. v_cvt_scalef32_pk_f16_fp4 turns two codes into fp16 (its
//    scale operand only contributes an exponent, so it is given 1.0) and
//    v_pk_mul_f16 applies the E4M3 scale, exactly. The power-of-two-only scale of the
//    gfx950 scaled MFMA cannot express an E4M3 scale, so it is not used.
//  - MXFP8: E4M3 * 2^e has 4 significant bits; v_cvt_scalef32_pk_bf16_fp8 applies
//    the E8M0 exponent while converting two codes to bf16, exactly. The scaled fp8
//    MFMA would take the codes directly, but its internal accumulation was measured
//    to lose about 200x more than fp32 accumulation (error ~1e-6 of sum |products|
//    versus ~1e-9 for the 16-bit MFMAs and for sequential fp32 FMA), which flips
//    intermediate codes and misses the output tolerance; so it is not used.
//
// Work item = (M-tile: BM consecutive sorted rows of one expert, N-tile of weight
// rows). The workgroup streams the N-tile's packed codes and block scales through LDS
// in K chunks with 16-byte global loads, loading chunk c into registers while chunk
// c-1 is multiplied out of LDS. K-slot mapping inside a 128-wide K group: lane group
// g = lane/16 holds k = 32g + 8j .. 32g + 8j + 7 for MFMA step j (both operands use
// it), so one step's weight bytes of a lane are one 32-bit (NVFP4) or 64-bit (MXFP8)
// LDS word inside a single scale block.
// gate_up tiles hold BN/2 gate rows and the BN/2 matching up rows, so the SwiGLU of the
// epilogue pairs two accumulators of the same lane.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

using namespace gemm_detail;

template <int FM, int BM, int BN, int KC, int WM, int WN, bool GATE_UP>
struct Cfg {
    static constexpr bool NV = FM == kFmtNV || FM == kFmtA16;  // NVFP4 weights
    static constexpr bool BW = FM == kFmtBF;                    // bf16 weights (no scales)
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MS = WTM / 16, NS = WTN / 16;
    static constexpr int BLK = NV ? 16 : 32;          // values per block scale
    static constexpr int B_ROW = NV ? KC / 2 : (BW ? 2 * KC : KC);  // code bytes per weight row per chunk
    static constexpr int SB = KC / BLK;               // scale bytes per weight row per chunk
    static constexpr int A_STRIDE = KC * 2 + 16;      // bytes per LDS A row (16-bit values)
    static constexpr int B_STRIDE = B_ROW + 16;
    static constexpr int A_OFF = 0;
    static constexpr int B_OFF = BM * A_STRIDE;
    static constexpr int S_OFF = B_OFF + BN * B_STRIDE;
    static constexpr int MAIN = S_OFF + BN * SB;
    static constexpr int EPI_STRIDE = BN / 2 + 4;     // floats per row of the MXFP8 SwiGLU tile
    static constexpr int EPI = (GATE_UP && FM == kFmtMX8) ? BM * EPI_STRIDE * 4 : 0;
    static constexpr int LDS = MAIN > EPI ? MAIN : EPI;
    static constexpr int A_TOTAL = BM * KC / 8;       // 16-byte loads of A per chunk
    static constexpr int A_ITEMS = (A_TOTAL + NT - 1) / NT;
    static constexpr int B_TOTAL = BN * B_ROW / 16;
    static constexpr int B_ITEMS = B_TOTAL / NT;
    static_assert(KC % 128 == 0, "K chunk must be whole 128-wide groups");
    static_assert(B_TOTAL % NT == 0, "B loads must tile the threads");
    static_assert(SB == 4 || SB == 8 || SB == 16, "scale row of 4, 8 or 16 bytes");
    static_assert(BN <= NT, "one scale load per weight row");
    static_assert(!GATE_UP || NS % 2 == 0, "gate and up halves");
};

template <int FM, int BM, int BN, int KC, int WM, int WN, bool GATE_UP>
__global__ void __launch_bounds__(WM * WN * 64) grouped_gemm_kernel(const GemmArgs p) {
    using C = Cfg<FM, BM, BN, KC, WM, WN, GATE_UP>;
    constexpr bool NV = C::NV;                   // NVFP4 weights (W4A4 or W4A16)
    constexpr bool BW = C::BW;                   // bf16 weights
    constexpr bool BF = FM != kFmtNV;            // bf16 operands and MFMA
    constexpr bool A16 = FM == kFmtA16;
    constexpr bool O16 = FM == kFmtA16 || FM == kFmtBF;  // bf16 intermediate out of gate_up
    using Frag = typename std::conditional<BF, bf16x8, half8>::type;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];

    const int tile = blockIdx.x;
    if (tile >= p.ctrl->n_tiles) return;
    const int el = p.tile_expert[tile];
    const int p0 = p.tile_row0[tile];
    const int rows = min(BM, p.offsets[el + 1] - p0);
    const int e = p.e_begin + el;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int r16 = lane & 15, g = lane >> 4;
    const int K = p.K;
    const int F = p.N / 2;  // gate_up only
    const int n0 = GATE_UP ? blockIdx.y * (BN / 2) : blockIdx.y * BN;
    const int64_t w_row_bytes = NV ? K / 2 : (BW ? 2 * K : K);

    // ---- per-thread global sources, fixed over the K loop
    const uint8_t *a_src[C::A_ITEMS];
    int a_dst[C::A_ITEMS];
#pragma unroll
    for (int i = 0; i < C::A_ITEMS; ++i) {
        const int item = tid + i * C::NT;
        const int r = item / (KC / 8), q = item % (KC / 8);
        a_dst[i] = item < C::A_TOTAL ? C::A_OFF + r * C::A_STRIDE + 16 * q : -1;
        a_src[i] = nullptr;
        if (item < C::A_TOTAL && r < rows) {
            const int pos = p0 + r;
            const int64_t arow = p.gather_by_token ? p.sorted_slot[pos] / p.top_k : pos;
            a_src[i] = static_cast<const uint8_t *>(p.a_vals) + arow * K * 2 + 16 * q;
        }
    }
    const uint8_t *b_src[C::B_ITEMS];
    int b_dst[C::B_ITEMS];
#pragma unroll
    for (int i = 0; i < C::B_ITEMS; ++i) {
        const int item = tid + i * C::NT;
        const int r = item / (C::B_ROW / 16), q = item % (C::B_ROW / 16);
        const int wrow = GATE_UP ? (r < BN / 2 ? n0 + r : F + n0 + (r - BN / 2)) : n0 + r;
        b_dst[i] = C::B_OFF + r * C::B_STRIDE + 16 * q;
        // packed tile layout (layout.h): a 16-byte piece stays inside one row's 64-wide slot
        b_src[i] = p.w_codes + (int64_t)e * p.N * w_row_bytes +
                   (BW ? layout::code_offset_bf16(K, wrow, 8 * q) : layout::code_offset(NV, K, wrow, (NV ? 32 : 16) * q));
    }
    const uint8_t *s_src = nullptr;
    int s_dst = 0;
    if (tid < BN && !BW) {
        const int wrow = GATE_UP ? (tid < BN / 2 ? n0 + tid : F + n0 + (tid - BN / 2)) : n0 + tid;
        s_src = p.w_scales + (int64_t)e * p.N * (K / C::BLK) + layout::scale_offset(NV, K, wrow, 0);
        s_dst = C::S_OFF + tid * C::SB;
    }

    // LDS B row of this lane in subtile ns
#define MOE_BROW(ns)                                                                                  \
    (GATE_UP ? ((ns) < C::NS / 2 ? wn * (C::WTN / 2) + 16 * (ns) + r16                                \
                                 : BN / 2 + wn * (C::WTN / 2) + 16 * ((ns) - C::NS / 2) + r16)        \
             : wn * C::WTN + 16 * (ns) + r16)

    float4_t acc[C::MS][C::NS];
#pragma unroll
    for (int i = 0; i < C::MS; ++i)
#pragma unroll
        for (int j = 0; j < C::NS; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

    u32x4 a_reg[C::A_ITEMS], b_reg[C::B_ITEMS];
    u32x4 s_reg = {0u, 0u, 0u, 0u};
    const int n_chunks = K / KC;
    for (int c = 0; c <= n_chunks; ++c) {
        if (c < n_chunks) {  // global -> registers for chunk c
            const int kn = c * KC;
#pragma unroll
            for (int i = 0; i < C::A_ITEMS; ++i)
                a_reg[i] = a_src[i] ? *reinterpret_cast<const u32x4 *>(a_src[i] + 2 * kn) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < C::B_ITEMS; ++i)
                b_reg[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + (int64_t)(kn / 64) *
                                                                       (BW ? 4096 : layout::code_block_bytes(NV)));
            if (s_src) {
                // the chunk's KC/64 block slots of this row, gathered in column order
                constexpr int NBLK = KC / 64, SBW = layout::scale_bytes_per_row(NV);
                const uint8_t *sp = s_src + (int64_t)(kn / 64) * layout::scale_block_bytes(NV);
                uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int b = 0; b < NBLK; ++b) {
                    const uint32_t v = SBW == 4 ? *reinterpret_cast<const uint32_t *>(sp + b * layout::scale_block_bytes(NV))
                                                : (uint32_t)*reinterpret_cast<const uint16_t *>(sp + b * layout::scale_block_bytes(NV));
                    if (SBW == 4) wv[b] = v;
                    else wv[b / 2] |= v << (16 * (b & 1));
                }
                s_reg = (u32x4){wv[0], wv[1], wv[2], wv[3]};
            }
        }
        if (c > 0) {  // multiply chunk c-1 out of LDS
#pragma unroll
            for (int jj = 0; jj < KC / 128; ++jj) {
                _Float16 sh[C::NS][2];
                float sf[C::NS][2];
                float sm[C::NS];
#pragma unroll
                for (int ns = 0; ns < C::NS; ++ns) {
                    const uint8_t *srow = smem + C::S_OFF + MOE_BROW(ns) * C::SB;
                    if (NV) {
                        // the two E4M3 scale bytes, exactly, by the hardware convert (unit scale)
                        const uint32_t two = *reinterpret_cast<const uint16_t *>(srow + 8 * jj + 2 * g);
                        const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two, 1.0f, false);
                        sh[ns][0] = h2[0];
                        sh[ns][1] = h2[1];
                        sf[ns][0] = (float)h2[0];
                        sf[ns][1] = (float)h2[1];
                    } else {
                        sm[ns] = __uint_as_float((uint32_t)srow[4 * jj + g] << 23);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kk = 128 * jj + 32 * g + 8 * j;  // k offset inside the chunk
                    Frag af[C::MS];
#pragma unroll
                    for (int ms = 0; ms < C::MS; ++ms)
                        af[ms] = *reinterpret_cast<const Frag *>(smem + C::A_OFF +
                                                                 (wm * C::WTM + 16 * ms + r16) * C::A_STRIDE + 2 * kk);
#pragma unroll
                    for (int ns = 0; ns < C::NS; ++ns) {
                        const uint8_t *brow = smem + C::B_OFF + MOE_BROW(ns) * C::B_STRIDE;
                        if constexpr (NV && !BF) {
                            const half8 bf = dequant_nvfp4(*reinterpret_cast<const uint32_t *>(brow + kk / 2),
                                                           sh[ns][j >> 1]);
#pragma unroll
                            for (int ms = 0; ms < C::MS; ++ms)
                                acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                        } else if constexpr (A16) {
                            const bf16x8 bf = dequant_nvfp4_bf16(*reinterpret_cast<const uint32_t *>(brow + kk / 2),
                                                                 sf[ns][j >> 1]);
#pragma unroll
                            for (int ms = 0; ms < C::MS; ++ms)
                                acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                        } else if constexpr (BW) {
                            const bf16x8 bf = *reinterpret_cast<const bf16x8 *>(brow + 2 * kk);  // the stored values
#pragma unroll
                            for (int ms = 0; ms < C::MS; ++ms)
                                acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                        } else {
                            const bf16x8 bf = dequant_mxfp8(*reinterpret_cast<const u32x2 *>(brow + kk), sm[ns]);
#pragma unroll
                            for (int ms = 0; ms < C::MS; ++ms)
                                acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                        }
                    }
                }
            }
        }
        __syncthreads();
        if (c < n_chunks) {  // registers -> LDS
#pragma unroll
            for (int i = 0; i < C::A_ITEMS; ++i)
                if (a_dst[i] >= 0) *reinterpret_cast<u32x4 *>(smem + a_dst[i]) = a_reg[i];
#pragma unroll
            for (int i = 0; i < C::B_ITEMS; ++i) *reinterpret_cast<u32x4 *>(smem + b_dst[i]) = b_reg[i];
            if (s_src) {
                if (C::SB == 16) *reinterpret_cast<u32x4 *>(smem + s_dst) = s_reg;
                else if (C::SB == 8) *reinterpret_cast<u32x2 *>(smem + s_dst) = (u32x2){s_reg.x, s_reg.y};
                else *reinterpret_cast<uint32_t *>(smem + s_dst) = s_reg.x;
            }
        }
        __syncthreads();
    }

    // ---- epilogue: C fragment of a lane = rows 4g..4g+3, column r16 of each 16x16 subtile
    const float sc = FM == kFmtNV ? p.a_tscale[0] * p.w_tscale[e] : (A16 ? p.w_tscale[e] : 1.0f);
    if (GATE_UP && FM == kFmtNV) {
        uint32_t amax = 0;
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < C::NS / 2; ++ns)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = wm * C::WTM + 16 * ms + 4 * g + i;
                    if (m >= rows) continue;
                    const int f = n0 + wn * (C::WTN / 2) + 16 * ns + r16;
                    const float hv = swiglu(acc[ms][ns][i] * sc, acc[ms][ns + C::NS / 2][i] * sc);
                    p.out_f32[(int64_t)(p0 + m) * F + f] = hv;
                    amax = max(amax, __float_as_uint(hv) & 0x7fffffffu);
                }
        for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
        if (lane == 0 && amax) atomic_max_grow(p.amax_bits, amax);
    } else if (GATE_UP && O16) {
        // W4A16 and bf16 experts: the SwiGLU output rounded to bf16 (nearest even) is the
        // down GEMM's input
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < C::NS / 2; ++ns)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = wm * C::WTM + 16 * ms + 4 * g + i;
                    if (m >= rows) continue;
                    const int64_t o = (int64_t)(p0 + m) * F + n0 + wn * (C::WTN / 2) + 16 * ns + r16;
                    const float hv = swiglu(acc[ms][ns][i] * sc, acc[ms][ns + C::NS / 2][i] * sc);
                    static_cast<__bf16 *>(p.o_vals)[o] = (__bf16)hv;
                    if (p.o_tap) p.o_tap[o] = hv;
                }
    } else if (GATE_UP) {
        // MXFP8: SwiGLU into an LDS tile [BM][BN/2], then quantise each 32-wide row block
        float *epi = reinterpret_cast<float *>(smem);
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < C::NS / 2; ++ns)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = wm * C::WTM + 16 * ms + 4 * g + i;
                    const int fl = wn * (C::WTN / 2) + 16 * ns + r16;
                    epi[m * C::EPI_STRIDE + fl] = swiglu(acc[ms][ns][i], acc[ms][ns + C::NS / 2][i]);
                }
        __syncthreads();
        constexpr int BLKS = (BN / 2) / 32;  // 32-blocks per tile row
        for (int item = tid; item < BM * BLKS; item += C::NT) {
            const int m = item / BLKS, q = item % BLKS;
            if (m >= rows) continue;
            float x[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] = epi[m * C::EPI_STRIDE + 32 * q + i];
            uint32_t cw[8];
            const int sc8 = mxfp8_quant_block(x, cw);
            const int64_t row = p0 + m;
            const int f = n0 + 32 * q;
            u32x4 *dst = reinterpret_cast<u32x4 *>(p.o_codes + row * F + f);
            dst[0] = (u32x4){cw[0], cw[1], cw[2], cw[3]};
            dst[1] = (u32x4){cw[4], cw[5], cw[6], cw[7]};
            p.o_scales[row * (F / 32) + f / 32] = (uint8_t)sc8;
            // exact bf16 values of the codes for the down GEMM
            store_dequant_mxfp8_32(static_cast<uint8_t *>(p.o_vals) + (row * F + f) * 2, cw, sc8);
            if (p.o_tap) {
                float4 *t = reinterpret_cast<float4 *>(p.o_tap + row * F + f);
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
            }
        }
    } else {
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < C::NS; ++ns)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = wm * C::WTM + 16 * ms + 4 * g + i;
                    if (m >= rows) continue;
                    const int n = n0 + wn * C::WTN + 16 * ns + r16;
                    p.out_f32[(int64_t)(p0 + m) * p.N + n] = NV ? acc[ms][ns][i] * sc : acc[ms][ns][i];
                }
    }
#undef MOE_BROW
}

template <int FM, int BM, int BN, int KC, int WM, int WN, bool GATE_UP>
hipError_t launch(const GemmArgs &a, int32_t max_tiles, hipStream_t s) {
    const int n_tiles_n = GATE_UP ? (a.N / 2) / (BN / 2) : a.N / BN;
    dim3 grid((unsigned)max_tiles, (unsigned)n_tiles_n);
    hipLaunchKernelGGL((grouped_gemm_kernel<FM, BM, BN, KC, WM, WN, GATE_UP>), grid, dim3(WM * WN * 64), 0, s, a);
    return hipGetLastError();
}

template <int FM>
hipError_t dispatch(const GemmArgs &a, bool gate_up, GemmShape shape, int32_t max_tiles, hipStream_t s) {
    if (shape == GemmShape::Decode) {
        if (a.K % 256 == 0)
            return gate_up ? launch<FM, 16, 128, 256, 1, 4, true>(a, max_tiles, s)
                           : launch<FM, 16, 128, 256, 1, 4, false>(a, max_tiles, s);
        return gate_up ? launch<FM, 16, 128, 128, 1, 4, true>(a, max_tiles, s)
                       : launch<FM, 16, 128, 128, 1, 4, false>(a, max_tiles, s);
    }
    return gate_up ? launch<FM, 128, 128, 128, 2, 2, true>(a, max_tiles, s)
                   : launch<FM, 128, 128, 128, 2, 2, false>(a, max_tiles, s);
}

}  // namespace

int32_t gemm_bm(GemmShape shape) { return shape == GemmShape::Decode ? 16 : 128; }

hipError_t launch_grouped_gemm(const GemmArgs &a, int fm, bool gate_up, GemmShape shape, int32_t max_tiles,
                               hipStream_t s) {
    switch (fm) {
        case kFmtNV: return dispatch<kFmtNV>(a, gate_up, shape, max_tiles, s);
        case kFmtMX8: return dispatch<kFmtMX8>(a, gate_up, shape, max_tiles, s);
        case kFmtA16: return dispatch<kFmtA16>(a, gate_up, shape, max_tiles, s);
        case kFmtBF: return dispatch<kFmtBF>(a, gate_up, shape, max_tiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
