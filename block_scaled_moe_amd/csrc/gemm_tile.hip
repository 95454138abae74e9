// gemm_tile.hip - grouped expert GEMMs for prefill-sized batches (many rows per expert),
// bound by the 16-bit MFMA rate.
//
// Same arithmetic as the other grouped GEMMs (exact 16-bit expansion of NVFP4 / MXFP8
// codes, fp32 accumulation; see gemm_common.h), tiled for MFMA throughput:
//  - workgroup tile 64 sorted rows x 256 weight rows, 4 waves side by side in N, each
//    wave 64 x 64 as 2 x 2 tiles of v_mfma_f32_32x32x16_{f16,bf16}; the waves share the
//    activation tile and own disjoint weight rows, so every weight value is expanded
//    once per workgroup;
//  - gate_up tiles hold 128 gate rows and the 128 matching up rows; wave w owns gate
//    rows 32w..32w+31 and the same up rows, so SwiGLU pairs two accumulators of a lane;
//  - K chunks of 64 go global -> registers (16-byte loads, next chunk prefetched while
//    the current one is multiplied) -> double-buffered LDS, one barrier per chunk;
//  - 64-row tiles keep the padding of ~170-row experts near 10%.
// 32x32x16 operand layout (measured on gfx950): A lane l holds row l%32, k 8(l/32)..+7;
// B lane l holds k 8(l/32)..+7 of column l%32; accumulator v of lane l is row
// 8(v/4) + 4(l/32) + v%4, column l%32. One 16-wide k step is one NVFP4 scale block and
// half an MXFP8 block.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace {

using namespace gemm_detail;

typedef float float16_t __attribute__((ext_vector_type(16)));

template <bool NV>
struct TileCfg {
    static constexpr int BM = 64, BN = 256, KC = 64, NT = 256;
    static constexpr int BLK = NV ? 16 : 32;
    static constexpr int B_ROW = NV ? KC / 2 : KC;     // code bytes per weight row per chunk
    static constexpr int SB = KC / BLK;                // scale bytes per weight row per chunk
    static constexpr int A_STRIDE = KC * 2 + 16;       // LDS bytes per activation row
    static constexpr int B_STRIDE = B_ROW + 16;        // LDS bytes per weight row
    static constexpr int A_OFF = 0;
    static constexpr int B_OFF = BM * A_STRIDE;
    static constexpr int S_OFF = B_OFF + BN * B_STRIDE;
    static constexpr int STAGE = S_OFF + BN * SB;
    static constexpr int A_ITEMS = BM * KC * 2 / 16 / NT;  // 16-byte loads per thread
    static constexpr int B_ITEMS = BN * B_ROW / 16 / NT;
    static_assert(BM * KC * 2 / 16 % NT == 0 && BN * B_ROW / 16 % NT == 0, "loads tile the threads");
    static_assert(SB == 2 || SB == 4, "one scale load per weight row");
};

template <bool NV, bool GATE_UP>
__global__ void __launch_bounds__(256, 2) tile_gemm_kernel(const GemmArgs p) {
    using C = TileCfg<NV>;
    using Frag = typename std::conditional<NV, half8, bf16x8>::type;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

    const int tile = blockIdx.x;
    if (tile >= p.ctrl->n_tiles) return;
    const int el = p.tile_expert[tile];
    const int p0 = p.tile_row0[tile];
    const int rows = min(C::BM, p.offsets[el + 1] - p0);
    const int e = p.e_begin + el;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g2 = lane >> 5;
    const int K = p.K, N = p.N, F = N / 2;
    const int n0 = GATE_UP ? blockIdx.y * (C::BN / 2) : blockIdx.y * C::BN;
    const int64_t w_row_bytes = NV ? K / 2 : K;

    // weight row of LDS tile row r
    auto wrow_of = [&](int r) -> int {
        return GATE_UP ? (r < C::BN / 2 ? n0 + r : F + n0 + (r - C::BN / 2)) : n0 + r;
    };

    // ---- per-thread global sources (fixed over K) and LDS destinations
    const uint8_t *a_src[C::A_ITEMS];
    int a_dst[C::A_ITEMS];
#pragma unroll
    for (int i = 0; i < C::A_ITEMS; ++i) {
        const int item = tid + i * C::NT;
        const int r = item / (C::KC * 2 / 16), q = item % (C::KC * 2 / 16);
        a_dst[i] = C::A_OFF + r * C::A_STRIDE + 16 * q;
        a_src[i] = nullptr;
        if (r < rows) {
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
        b_dst[i] = C::B_OFF + r * C::B_STRIDE + 16 * q;
        b_src[i] = p.w_codes + ((int64_t)e * N + wrow_of(r)) * w_row_bytes + 16 * q;
    }
    const uint8_t *s_src = p.w_scales + ((int64_t)e * N + wrow_of(tid)) * (K / C::BLK);
    const int s_dst = C::S_OFF + tid * C::SB;

    // LDS weight row of this lane in its wave's subtile ns (0, 1)
    const int brow0 = GATE_UP ? 32 * wave + l32 : 64 * wave + l32;
    const int brow1 = GATE_UP ? C::BN / 2 + 32 * wave + l32 : 64 * wave + 32 + l32;

    float16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (float16_t){};

    u32x4 a_reg[C::A_ITEMS], b_reg[C::B_ITEMS];
    uint32_t s_reg = 0;
    const int n_chunks = K / C::KC;
    auto load = [&](int c) {
        const int kn = c * C::KC;
#pragma unroll
        for (int i = 0; i < C::A_ITEMS; ++i)
            a_reg[i] = a_src[i] ? *reinterpret_cast<const u32x4 *>(a_src[i] + 2 * kn) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < C::B_ITEMS; ++i)
            b_reg[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + (NV ? kn / 2 : kn));
        s_reg = C::SB == 4 ? *reinterpret_cast<const uint32_t *>(s_src + kn / C::BLK)
                           : (uint32_t)*reinterpret_cast<const uint16_t *>(s_src + kn / C::BLK);
    };
    auto store = [&](int buf) {
        uint8_t *base = smem + buf * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_ITEMS; ++i) *reinterpret_cast<u32x4 *>(base + a_dst[i]) = a_reg[i];
#pragma unroll
        for (int i = 0; i < C::B_ITEMS; ++i) *reinterpret_cast<u32x4 *>(base + b_dst[i]) = b_reg[i];
        if (C::SB == 4) *reinterpret_cast<uint32_t *>(base + s_dst) = s_reg;
        else *reinterpret_cast<uint16_t *>(base + s_dst) = (uint16_t)s_reg;
    };

    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
        if (c + 1 < n_chunks) load(c + 1);
        const uint8_t *base = smem + (c & 1) * C::STAGE;
#pragma unroll
        for (int st = 0; st < C::KC / 16; ++st) {
            const int kk = 16 * st + 8 * g2;  // this lane's k inside the chunk
            Frag af[2];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
                af[ms] = *reinterpret_cast<const Frag *>(base + C::A_OFF + (32 * ms + l32) * C::A_STRIDE + 2 * kk);
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const int row = ns ? brow1 : brow0;
                const uint8_t *brow = base + C::B_OFF + row * C::B_STRIDE;
                const uint8_t sc = base[C::S_OFF + row * C::SB + (NV ? st : st / 2)];
                if constexpr (NV) {
                    const half8 bf = dequant_nvfp4(*reinterpret_cast<const uint32_t *>(brow + kk / 2), e4m3_to_f16(sc));
#pragma unroll
                    for (int ms = 0; ms < 2; ++ms)
                        acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                } else {
                    const bf16x8 bf = dequant_mxfp8(*reinterpret_cast<const u32x2 *>(brow + kk),
                                                    __uint_as_float((uint32_t)sc << 23));
#pragma unroll
                    for (int ms = 0; ms < 2; ++ms)
                        acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                }
            }
        }
        if (c + 1 < n_chunks) store((c + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: accumulator v of lane l = row 8(v/4) + 4 g2 + v%4 (+32 ms), column l32
    const float scl = NV ? p.a_tscale[0] * p.w_tscale[e] : 1.0f;
    if (GATE_UP) {
        const int f = n0 + 32 * wave + l32;
        uint32_t amax = 0;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                const float hv = swiglu(acc[ms][0][v] * scl, acc[ms][1][v] * scl);
                if (NV) {
                    if (m < rows) {
                        p.out_f32[(int64_t)(p0 + m) * F + f] = hv;
                        amax = max(amax, __float_as_uint(hv) & 0x7fffffffu);
                    }
                } else {
                    // MXFP8: the 32 columns of row m (one block) are the 32 lanes of this half-wave
                    float a = fabsf(hv);
#pragma unroll
                    for (int off = 16; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
                    const int sc8 = e8m0_code_for_amax(a);
                    const int code = e4m3_encode(ldexpf(hv, -(sc8 - 127)));
                    if (m < rows) {
                        const int64_t row = p0 + m;
                        p.o_codes[row * F + f] = (uint8_t)code;
                        const float s2 = ldexpf(1.0f, sc8 - 127);
                        static_cast<uint16_t *>(p.o_vals)[row * F + f] =
                            (uint16_t)((__float_as_uint(e4m3_value_pos(code & 0x7f) * s2) >> 16) |
                                       ((uint32_t)(code & 0x80) << 8));
                        if (l32 == 0) p.o_scales[row * (F / 32) + (n0 + 32 * wave) / 32] = (uint8_t)sc8;
                        if (p.o_tap) p.o_tap[row * F + f] = hv;
                    }
                }
            }
        }
        if (NV) {
            for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
            if (lane == 0 && amax) atomicMax(p.amax_bits, amax);
        }
    } else {
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const int n = n0 + 64 * wave + 32 * ns + l32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                    if (m < rows) p.out_f32[(int64_t)(p0 + m) * N + n] = NV ? acc[ms][ns][v] * scl : acc[ms][ns][v];
                }
            }
    }
}

template <bool NV, bool GATE_UP>
hipError_t launch_t(const GemmArgs &a, int32_t max_tiles, hipStream_t s) {
    using C = TileCfg<NV>;
    const int n_tiles_n = GATE_UP ? (a.N / 2) / (C::BN / 2) : a.N / C::BN;
    hipLaunchKernelGGL((tile_gemm_kernel<NV, GATE_UP>), dim3((unsigned)max_tiles, (unsigned)n_tiles_n), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace

bool tile_gemm_supported(int32_t K, int32_t N, bool gate_up) {
    return K % 64 == 0 && (gate_up ? (N / 2) % 128 == 0 : N % 256 == 0);
}

hipError_t launch_tile_gemm(const GemmArgs &a, bool nvfp4, bool gate_up, int32_t max_tiles, hipStream_t s) {
    if (nvfp4) return gate_up ? launch_t<true, true>(a, max_tiles, s) : launch_t<true, false>(a, max_tiles, s);
    return gate_up ? launch_t<false, true>(a, max_tiles, s) : launch_t<false, false>(a, max_tiles, s);
}

}  // namespace moe
