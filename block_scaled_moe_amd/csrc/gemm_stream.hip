// gemm_stream.hip - grouped expert GEMMs for decode-sized batches: few rows per expert,
// so the layer is bound by streaming the packed expert weights from HBM once.
//
// Same arithmetic as the tiled kernels (exact 16-bit expansion of NVFP4 / MXFP8 codes,
// 16x16x32 MFMA, fp32 accumulation; see gemm_common.h; for W4A16 the NVFP4 weights are
// expanded to bf16 and the activations are the bf16 values), organised for bandwidth:
//  - a workgroup owns one M-tile (<= 16 sorted rows of one expert) and 64 weight rows
//    (gate_up: 32 gate rows and the 32 matching up rows; down: 64 output columns);
//  - its 4 waves split K into quarters, and each lane streams its weight bytes straight
//    from HBM into registers in the MFMA operand layout (16-byte loads; the 4 lanes of a
//    row cover 64 contiguous bytes per NVFP4 group, 128 per MXFP8 group), keeping a
//    window of W groups of loads in flight; nothing goes through LDS and the K loop has
//    no barriers;
//  - weights are in the packed tile layout (layout.h), so the 16 rows x 4 lanes of one
//    load instruction read two contiguous 512-byte (NVFP4) runs;
//  - the wave's block scales are staged once in LDS with contiguous loads;
//  - the four partial sums are added in a fixed order through LDS before the epilogue,
//    so results are deterministic.
// K-slot mapping inside a 128-wide group of a wave's K quarter (two 64-wide chunks of the
// tile layout), chosen so that one weight load instruction of a wave reads whole rows of
// a chunk: lane group g = lane/16 holds, for MFMA step j, the 8 values at
//   NVFP4  k = 32g + 8j                        (one 16-byte load: chunk g/2, half g%2)
//   MXFP8  k = 64(j/2) + 16g + 8(j%2)          (load q = j/2: quarter g of chunk q)
//   bf16   k = 64(j/2) + 32(j%2) + 8g          (load q = j: bytes 16g.. of half q%2 of chunk q/2)
// (a summation-order permutation only); the activation fragment of lane (row r, g) is
// read at the same k from the exact 16-bit activation row.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

using namespace gemm_detail;

typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kSub = 4;    // 16-row weight subtiles per workgroup
constexpr int kRows = 64;  // weight rows per workgroup

// Tuning: K groups of weight loads in flight per wave, and the occupancy (waves per SIMD)
// the register budget is set for. A workgroup streams one panel and exits, so its start
// (first loads in flight) and end (cross-wave sum, epilogue) leave its slot idle; more
// resident workgroups per CU cover those phases. Measured on the NVFP4 decode layer: two
// groups at three waves per SIMD beat four groups at two (gate_up 0.536 -> 0.498 ms,
// down 0.287 -> 0.270 ms); three groups at three waves spill and lose; one group at four
// waves matches two at three on NVFP4 and is 3% faster on W4A16 (more expansion VALU
// per byte to hide). MXFP8 (twice the
// bytes per lane) keeps two groups at two waves (one group at three measured slower);
// bf16 takes one group at two waves (2% faster than two groups at one).
#ifndef MOE_STREAM_W_NV
#define MOE_STREAM_W_NV 1
#endif
#ifndef MOE_STREAM_W_MX
#define MOE_STREAM_W_MX 2
#endif
#ifndef MOE_STREAM_W_BF
#define MOE_STREAM_W_BF 1
#endif
#ifndef MOE_STREAM_OCC_NV
#define MOE_STREAM_OCC_NV 4
#endif
#ifndef MOE_STREAM_OCC_MX
#define MOE_STREAM_OCC_MX 2
#endif
#ifndef MOE_STREAM_OCC_BF
#define MOE_STREAM_OCC_BF 2
#endif
template <int FM>
constexpr int stream_occupancy() {
    return (FM == kFmtNV || FM == kFmtA16) ? MOE_STREAM_OCC_NV : (FM == kFmtMX8 ? MOE_STREAM_OCC_MX : MOE_STREAM_OCC_BF);
}

// weight loads: at decode each (expert, weight row) panel is read by one workgroup exactly
// once, so where one load instruction covers whole cache lines (NVFP4: 16 rows x 64
// bytes of two chunks; MXFP8: 16 rows x 16 bytes of each quarter of one chunk; bf16:
// 16 rows x 64 bytes of one half-chunk) they can be marked non-temporal, which measured
// 3-6% faster on NVFP4 and 13% on MXFP8.
#ifndef MOE_STREAM_NT_MX
#define MOE_STREAM_NT_MX 1
#endif
#ifndef MOE_STREAM_NT_BF
#define MOE_STREAM_NT_BF 1
#endif
template <bool NT>
__device__ __forceinline__ u32x4 load_w(const u32x4 *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <int FM, bool GATE_UP, int G>  // G = 128-wide K groups per wave (K = 512 G)
__global__ void __launch_bounds__(256, (stream_occupancy<FM>())) stream_gemm_kernel(const GemmArgs p) {
    constexpr bool NV = FM == kFmtNV || FM == kFmtA16;  // NVFP4 weights (W4A4 or W4A16)
    constexpr bool BW = FM == kFmtBF;                    // bf16 weights (no scales)
    constexpr bool BF = FM != kFmtNV;                    // bf16 operands and MFMA
    constexpr bool A16 = FM == kFmtA16;
    constexpr bool O16 = FM == kFmtA16 || FM == kFmtBF;  // bf16 intermediate out of gate_up
    using Frag = typename std::conditional<BF, bf16x8, half8>::type;
    constexpr int NQ = NV ? 1 : (BW ? 4 : 2);      // 16-byte code loads per lane, group and subtile
    constexpr int W = NV ? MOE_STREAM_W_NV : (BW ? MOE_STREAM_W_BF : MOE_STREAM_W_MX);  // groups of loads in flight
    constexpr int BLK = NV ? 16 : 32;
    constexpr int SBW = G * 128 / BLK;             // scale bytes per weight row in a wave's K quarter
    __shared__ __attribute__((aligned(16))) uint8_t s_scale[4][kRows * SBW];
    __shared__ __attribute__((aligned(16))) float s_red[4][kSub][64][4];
    __shared__ float s_epi[16][33];                // MXFP8 gate_up: SwiGLU tile, 16 rows x 32 f

    const int tile = blockIdx.y;  // the slow grid axis: see launch_g
    if (tile >= p.ctrl->n_tiles) return;
    const int el = p.tile_expert[tile];
    const int p0 = p.tile_row0[tile];
    const int rows = min(16, p.offsets[el + 1] - p0);
    const int e = p.e_begin + el;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int K = p.K;
    const int F = p.N / 2;
    const int n0 = GATE_UP ? blockIdx.x * (kRows / 2) : blockIdx.x * kRows;
    const int kw = wave * G * 128;  // first k of this wave's quarter
    const int64_t row_bytes = NV ? K / 2 : (BW ? 2 * K : K);

    auto wrow_of = [&](int r) -> int {  // weight row of tile row r (0..63)
        return GATE_UP ? (r < kRows / 2 ? n0 + r : F + n0 + (r - kRows / 2)) : n0 + r;
    };

    // packed tile layout (layout.h): rows in groups of 32, K in blocks of 64
    constexpr int CB = BW ? 128 : layout::code_bytes_per_row(NV);
    constexpr int CBLK = 32 * CB, SBLK = layout::scale_block_bytes(NV);
    const int64_t kb = K / 64;
    const uint8_t *w_codes_e = p.w_codes + (int64_t)e * p.N * row_bytes;
    const uint8_t *w_scales_e = p.w_scales + (int64_t)e * p.N * (K / BLK);

    // ---- block scales of this wave's quarter: global -> registers now, -> LDS (row-major,
    //      SBW bytes per row) after the first weight loads are in flight. Register i of
    //      lane l: NVFP4 row l's 4 scales of chunk i; MXFP8 rows 2(l%32), 2(l%32)+1 of chunk
    //      2i + l/32 (consecutive lanes read consecutive bytes of one block).
    constexpr int SREG = kRows * SBW / 4 / 64;
    static_assert(kRows * SBW / 4 % 64 == 0, "scale dwords tile the wave");
    uint32_t sreg[SREG];
#pragma unroll
    for (int i = 0; i < SREG; ++i) {
        if (BW) {
            sreg[i] = 0;  // no scales
        } else if (NV) {
            const int r = lane, row = wrow_of(r);
            sreg[i] = *reinterpret_cast<const uint32_t *>(w_scales_e + ((row >> 5) * kb + kw / 64 + i) * SBLK +
                                                          4 * (row & 31));
        } else {
            const int r = 2 * (lane & 31), row = wrow_of(r), cl = 2 * i + (lane >> 5);
            sreg[i] = *reinterpret_cast<const uint32_t *>(w_scales_e + ((row >> 5) * kb + kw / 64 + cl) * SBLK +
                                                          2 * (row & 31));
        }
    }

    // ---- weight code pointers of this lane (one per subtile, at its first load of the
    //      wave's first group; see the K mapping in the header) and activation row
    const uint8_t *bsrc[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
        const int row = wrow_of(16 * s + r16);
        bsrc[s] = w_codes_e + ((row >> 5) * kb + kw / 64) * CBLK +
                  (NV ? (row & 31) * CB + (g >> 1) * CBLK + (CB / 2) * (g & 1)
                      : (BW ? (row & 31) * 64 + 16 * g : 512 * g + (row & 31) * 16));
    }
    // byte offset of load q of a group from the lane's pointer
    auto wq_off = [&](int q) -> int { return NV ? 0 : (BW ? (q >> 1) * CBLK + 2048 * (q & 1) : q * CBLK); };
    // k of MFMA step j inside a group, for lane group g
    auto k_of = [&](int j) -> int {
        return NV ? 32 * g + 8 * j : (BW ? 64 * (j >> 1) + 32 * (j & 1) + 8 * g : 64 * (j >> 1) + 16 * g + 8 * (j & 1));
    };
    const uint8_t *asrc = nullptr;
    if (r16 < rows) {
        const int pos = p0 + r16;
        const int64_t arow = p.gather_by_token ? p.sorted_slot[pos] / p.top_k : pos;
        asrc = static_cast<const uint8_t *>(p.a_vals) + (arow * K + kw) * 2;
    }

    u32x4 bq[G][kSub][NQ];
    u32x4 aq[G][4];
    auto load_group = [&](int jj) {
#pragma unroll
        for (int s = 0; s < kSub; ++s)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                bq[jj][s][q] = load_w<NV || (BW ? MOE_STREAM_NT_BF : MOE_STREAM_NT_MX)>(
                    reinterpret_cast<const u32x4 *>(bsrc[s] + 2 * CBLK * jj + wq_off(q)));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            aq[jj][j] = asrc ? *reinterpret_cast<const u32x4 *>(asrc + 256 * jj + 2 * k_of(j)) : (u32x4){0u, 0u, 0u, 0u};
    };

    float4_t acc[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) acc[s] = (float4_t){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int jj = 0; jj < W && jj < G; ++jj) load_group(jj);
#pragma unroll
    for (int i = 0; i < SREG; ++i) {
        if (BW) {
        } else if (NV) {
            *reinterpret_cast<uint32_t *>(&s_scale[wave][lane * SBW + 4 * i]) = sreg[i];
        } else {
            const int r = 2 * (lane & 31), cl = 2 * i + (lane >> 5);
            *reinterpret_cast<uint16_t *>(&s_scale[wave][r * SBW + 2 * cl]) = (uint16_t)sreg[i];
            *reinterpret_cast<uint16_t *>(&s_scale[wave][(r + 1) * SBW + 2 * cl]) = (uint16_t)(sreg[i] >> 16);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's scale stores are done
    __builtin_amdgcn_wave_barrier();     // and no LDS read is hoisted above them

#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
        if (jj + W < G) load_group(jj + W);
        _Float16 sh[kSub][2];
        float sf[kSub][2];
        float sm[kSub][2];
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
            const uint8_t *srow = &s_scale[wave][(16 * s + r16) * SBW];
            if (BW) {
                sm[s][0] = sm[s][1] = 1.0f;
            } else if (NV) {
                // the two E4M3 scale bytes, exactly, by the hardware convert (unit scale)
                const uint32_t two = *reinterpret_cast<const uint16_t *>(srow + 8 * jj + 2 * g);
                if constexpr (A16) {
                    const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(two, 1.0f, false);
                    sf[s][0] = f2[0];
                    sf[s][1] = f2[1];
                } else {
                    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two, 1.0f, false);
                    sh[s][0] = h2[0];
                    sh[s][1] = h2[1];
                }
            } else {
                // steps 2h, 2h + 1 lie in 32-block 2h + g/2 of the group
                sm[s][0] = __uint_as_float((uint32_t)srow[4 * jj + (g >> 1)] << 23);
                sm[s][1] = __uint_as_float((uint32_t)srow[4 * jj + 2 + (g >> 1)] << 23);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const Frag af = __builtin_bit_cast(Frag, aq[jj][j]);
#pragma unroll
            for (int s = 0; s < kSub; ++s) {
                if constexpr (NV && !BF) {
                    const half8 bf = dequant_nvfp4(bq[jj][s][0][j], sh[s][j >> 1]);
                    acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[s], 0, 0, 0);
                } else if constexpr (A16) {
                    const bf16x8 bf = dequant_nvfp4_bf16(bq[jj][s][0][j], sf[s][j >> 1]);
                    acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[s], 0, 0, 0);
                } else if constexpr (BW) {
                    const bf16x8 bf = __builtin_bit_cast(bf16x8, bq[jj][s][j]);  // the stored values
                    acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[s], 0, 0, 0);
                } else {
                    const u32x4 w4 = bq[jj][s][j >> 1];
                    const u32x2 w2 = (j & 1) ? (u32x2){w4.z, w4.w} : (u32x2){w4.x, w4.y};
                    const bf16x8 bf = dequant_mxfp8(w2, sm[s][j >> 1]);
                    acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[s], 0, 0, 0);
                }
            }
        }
    }

    // ---- cross-wave reduction in a fixed order, then the epilogue
#pragma unroll
    for (int s = 0; s < kSub; ++s)
        *reinterpret_cast<float4_t *>(&s_red[wave][s][lane][0]) = acc[s];
    __syncthreads();
    auto reduced = [&](int s) -> float4_t {
        float4_t v = *reinterpret_cast<const float4_t *>(&s_red[0][s][lane][0]);
#pragma unroll
        for (int w = 1; w < 4; ++w) v += *reinterpret_cast<const float4_t *>(&s_red[w][s][lane][0]);
        return v;
    };
    const float sc = FM == kFmtNV ? p.a_tscale[0] * p.w_tscale[e] : (A16 ? p.w_tscale[e] : 1.0f);
    if (GATE_UP) {
        // waves 0 and 1: gate subtile w with up subtile w + 2 (16 f columns each)
        if (wave < 2) {
            const float4_t gv = reduced(wave), uv = reduced(wave + 2);
            const int fl = 16 * wave + r16;  // f inside the tile
            uint32_t amax = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * g + i;
                const float hv = swiglu(gv[i] * sc, uv[i] * sc);
                if (O16) {
                    // the SwiGLU output rounded to bf16 (nearest even) is the down GEMM's input
                    if (m < rows) {
                        const int64_t o = (int64_t)(p0 + m) * F + n0 + fl;
                        static_cast<__bf16 *>(p.o_vals)[o] = (__bf16)hv;
                        if (p.o_tap) p.o_tap[o] = hv;
                    }
                } else if (NV) {
                    if (m < rows) {
                        p.out_f32[(int64_t)(p0 + m) * F + n0 + fl] = hv;
                        amax = max(amax, __float_as_uint(hv) & 0x7fffffffu);
                    }
                } else {
                    s_epi[m][fl] = hv;
                }
            }
            if (FM == kFmtNV) {
                for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
                if (lane == 0 && amax) atomic_max_grow(p.amax_bits, amax);
            }
        }
        if (FM == kFmtMX8) {
            __syncthreads();
            // one 32-block of the MXFP8 intermediate per tile row
            const int m = threadIdx.x;
            if (m < rows) {
                float x[32];
#pragma unroll
                for (int i = 0; i < 32; ++i) x[i] = s_epi[m][i];
                uint32_t cw[8];
                const int sc8 = mxfp8_quant_block(x, cw);
                const int64_t row = p0 + m;
                u32x4 *dst = reinterpret_cast<u32x4 *>(p.o_codes + row * F + n0);
                dst[0] = (u32x4){cw[0], cw[1], cw[2], cw[3]};
                dst[1] = (u32x4){cw[4], cw[5], cw[6], cw[7]};
                p.o_scales[row * (F / 32) + n0 / 32] = (uint8_t)sc8;
                store_dequant_mxfp8_32(static_cast<uint8_t *>(p.o_vals) + (row * F + n0) * 2, cw, sc8);
                if (p.o_tap) {
                    float4 *t = reinterpret_cast<float4 *>(p.o_tap + row * F + n0);
#pragma unroll
                    for (int i = 0; i < 8; ++i) t[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
                }
            }
        }
    } else {
        // wave w writes output subtile w (16 columns)
        const float4_t v = reduced(wave);
        const int n = n0 + 16 * wave + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < rows) p.out_f32[(int64_t)(p0 + m) * p.N + n] = NV ? v[i] * sc : v[i];
        }
    }
}

// The grid covers the host's bound on the M-tiles (max_tiles; the device's count is
// ctrl->n_tiles, about 70% of it at decode). With the tile on the slow axis the
// workgroups of tiles past the count come after all the real ones instead of among them:
// decode-nvfp4 gate_up 0.502 -> 0.496 ms, down 0.269 -> 0.256 ms.
template <int FM, bool GATE_UP, int G>
hipError_t launch_g(const GemmArgs &a, int32_t max_tiles, hipStream_t s) {
    const int n_tiles_n = GATE_UP ? (a.N / 2) / (kRows / 2) : a.N / kRows;
    // decode shapes (fewer than 48 slots per expert, at most 4096 experts) bound max_tiles
    // far below the 65535 limit of the y axis
    if (max_tiles > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((stream_gemm_kernel<FM, GATE_UP, G>), dim3((unsigned)n_tiles_n, (unsigned)max_tiles),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int FM, bool GATE_UP>
hipError_t launch_k(const GemmArgs &a, int32_t max_tiles, hipStream_t s) {
    switch (a.K / 512) {
        case 1: return launch_g<FM, GATE_UP, 1>(a, max_tiles, s);
        case 2: return launch_g<FM, GATE_UP, 2>(a, max_tiles, s);
        case 3: return launch_g<FM, GATE_UP, 3>(a, max_tiles, s);
        case 4: return launch_g<FM, GATE_UP, 4>(a, max_tiles, s);
        case 5: return launch_g<FM, GATE_UP, 5>(a, max_tiles, s);
        case 6: return launch_g<FM, GATE_UP, 6>(a, max_tiles, s);
        case 7: return launch_g<FM, GATE_UP, 7>(a, max_tiles, s);
        case 8: return launch_g<FM, GATE_UP, 8>(a, max_tiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool stream_gemm_supported(int32_t K, int32_t N, bool gate_up) {
    return K % 512 == 0 && K / 512 >= 1 && K / 512 <= 8 && (gate_up ? (N / 2) % 32 == 0 : N % 64 == 0);
}

hipError_t launch_stream_gemm(const GemmArgs &a, int fm, bool gate_up, int32_t max_tiles, hipStream_t s) {
    switch (fm) {
        case kFmtNV: return gate_up ? launch_k<kFmtNV, true>(a, max_tiles, s) : launch_k<kFmtNV, false>(a, max_tiles, s);
        case kFmtMX8: return gate_up ? launch_k<kFmtMX8, true>(a, max_tiles, s) : launch_k<kFmtMX8, false>(a, max_tiles, s);
        case kFmtA16: return gate_up ? launch_k<kFmtA16, true>(a, max_tiles, s) : launch_k<kFmtA16, false>(a, max_tiles, s);
        case kFmtBF: return gate_up ? launch_k<kFmtBF, true>(a, max_tiles, s) : launch_k<kFmtBF, false>(a, max_tiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
