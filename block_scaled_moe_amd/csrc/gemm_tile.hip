// gemm_tile.hip - grouped expert GEMMs for prefill-sized batches (many rows per expert),
// bound by the 16-bit MFMA rate.
//
// Same arithmetic as the other grouped GEMMs (exact 16-bit expansion of NVFP4 / MXFP8
// codes, fp32 accumulation; see gemm_common.h), tiled for MFMA throughput:
//  - workgroup tile BM sorted rows x (128 NS) weight rows, 4 waves side by side in N,
//    each wave BM x 32NS as BM/32 x NS tiles of v_mfma_f32_32x32x16_{f16,bf16}; per
//    format (tile_bm, tile_ns) BM = 64, NS = 4 for NVFP4 and W4A16, BM = 128, NS = 2 for
//    MXFP8, BM = 64, NS = 2 for bf16. Per MFMA a wave issues 256 / BM expansion
//    instructions (NVFP4) and 1/NS activation reads from LDS; the shapes are the measured
//    best trade between the two at the register budget of two or three waves per SIMD;
//  - a tile runs only the 32-row M-subtiles that hold rows (short tiles);
//  - the waves own disjoint weight rows, so weights never pass through LDS: each lane
//    loads its weight row's codes straight into registers and expands them into the
//    MFMA B operand; only the shared activation tile is staged in LDS;
//  - K order inside a 64-wide chunk is permuted identically for both operands: lane half
//    g (lanes 32g..32g+31) supplies k = 32g..32g+31 over the chunk's four MFMA steps
//    (step s: k = 32g + 8s .. +7). With the packed tile layout (layout.h) a wave's codes
//    for one chunk and 32-row subtile are then one contiguous 1 KiB (NVFP4) / 2 KiB
//    (MXFP8: two 512-byte runs per load instruction, its quarters being apart) and its
//    scales one 128 / 64-byte run; the fp32 sums are unchanged up to rounding order;
//  - software pipeline without branches: activations two chunks ahead (two register
//    sets, LDS double buffer), weights WR chunks ahead (register ring), so every wait
//    count in the loop is partial; a two-slot ring measured faster than deeper rings at
//    fewer waves per SIMD;
//  - gate_up tiles pair gate row f with up row F + f in the same lane and accumulator
//    slot, so SwiGLU needs no data exchange;
//  - work items (M-tile, N-block) are ordered expert-major (gemm_common.h) and dealt to
//    the 8 XCDs in contiguous ranges, so one XCD's L2 serves an expert's weight panel to
//    all of its M-tiles and the activation rows of those tiles across its N-blocks.
// 32x32x16 operand layout (measured on gfx950): A lane l holds row l%32, k 8(l/32)..+7;
// B lane l holds k 8(l/32)..+7 of column l%32; accumulator v of lane l is row
// 8(v/4) + 4(l/32) + v%4, column l%32.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

using namespace gemm_detail;

typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kKC = 64, kThreads = 256, kGroup = 4;
constexpr int kAStride = kKC * 2 + 16;  // LDS bytes per activation row

// rows per M-tile: 128 for NVFP4 W4A4 and MXFP8 (each expanded weight fragment feeds four
// 32-row MFMAs, halving the expansion VALU per MFMA), 64 for the others
#ifndef MOE_TILE_BM_NV
#define MOE_TILE_BM_NV 64
#endif
#ifndef MOE_TILE_BM_MX
#define MOE_TILE_BM_MX 128
#endif
#ifndef MOE_TILE_BM_BF
#define MOE_TILE_BM_BF 64
#endif
#ifndef MOE_TILE_BM_A16
#define MOE_TILE_BM_A16 64
#endif
template <int FM>
constexpr int tile_bm() {
    return FM == kFmtNV ? MOE_TILE_BM_NV
                        : (FM == kFmtMX8 ? MOE_TILE_BM_MX : (FM == kFmtBF ? MOE_TILE_BM_BF : MOE_TILE_BM_A16));
}
template <int BM>
constexpr int a_stage() { return BM * kAStride; }  // one LDS activation buffer
template <int BM>
constexpr int a_items() { return BM * kKC * 2 / 16 / kThreads; }  // 16-byte activation loads per thread
static_assert(64 * kKC * 2 / 16 % kThreads == 0, "activation loads tile the threads");

#ifndef MOE_TILE_WR
#define MOE_TILE_WR 2  // weight chunks in flight (register ring slots)
#endif
// The loop picks the activation register set and LDS buffer of chunk c = c0 + j by j & 1,
// which equals c & 1 only while c0 (a multiple of the ring size) is even.
static_assert(MOE_TILE_WR % 2 == 0, "the weight ring size must be even");
#ifndef MOE_TILE_SHORT
#define MOE_TILE_SHORT 1  // short tiles run only the M-subtiles holding rows
#endif
#ifndef MOE_TILE_NS_NV
#define MOE_TILE_NS_NV (MOE_TILE_BM_NV == 128 ? 2 : 4)
#endif
#ifndef MOE_TILE_NS_MX
#define MOE_TILE_NS_MX 2
#endif
#ifndef MOE_TILE_NS_A16
#define MOE_TILE_NS_A16 4
#endif

// 32-row weight subtiles per wave in N: 2 with 128-row tiles (128 accumulator registers,
// two waves per SIMD); with 64-row tiles NVFP4 4 (its expansion costs twice MXFP8's
// VALU, so each activation fragment feeds more MFMAs; 234 registers, two waves per SIMD),
// MXFP8 2 (three waves per SIMD; at 4 it spills), W4A16 as NVFP4
template <int FM>
constexpr int tile_ns() {
    return (FM == kFmtMX8 || FM == kFmtBF) ? MOE_TILE_NS_MX : (FM == kFmtNV ? MOE_TILE_NS_NV : MOE_TILE_NS_A16);
}

// floats per row of a wave's MXFP8 epilogue tile in LDS: 16 NS columns plus one, so
// lanes reading rows at the same column fall on different banks
template <int NS>
constexpr int kEpiStride() { return 16 * NS + 1; }
// floats per row of a wave's 32 x 32 output staging tile (16-byte rows; four waves' tiles
// fit the smallest activation double buffer)
constexpr int kYStride = 36;

__device__ __forceinline__ void store_f4(float *p, float4 v, bool nt) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v x = {v.x, v.y, v.z, v.w};
    if (nt)
        __builtin_nontemporal_store(x, reinterpret_cast<f4v *>(p));
    else
        *reinterpret_cast<f4v *>(p) = x;
}

// LDS of one workgroup: the double-buffered activation tile, or for the MXFP8 gate_up
// epilogue the four waves' SwiGLU tiles if larger
template <int FM, bool GATE_UP, int NS, int BM>
constexpr int tile_smem_bytes() {
    return (FM == kFmtMX8 && GATE_UP && 4 * BM * kEpiStride<NS>() * 4 > 2 * a_stage<BM>()) ? 4 * BM * kEpiStride<NS>() * 4
                                                                                     : 2 * a_stage<BM>();
}

// waves per SIMD the register budget is set for
template <int NS, int BM>
constexpr int tile_waves_per_simd() { return BM == 64 ? (NS == 2 ? 3 : 2) : (NS == 2 ? 2 : 1); }

template <int FM, bool GATE_UP, int NS, int BM>
__global__ void __launch_bounds__(kThreads, (tile_waves_per_simd<NS, BM>())) tile_gemm_kernel(const GemmArgs p) {
    constexpr int kBM = BM, kMS = BM / 32;  // rows per M-tile, 32-row MFMA subtiles per wave
    constexpr int kAStage = a_stage<BM>(), kAItems = a_items<BM>();
    constexpr bool NV = FM == kFmtNV || FM == kFmtA16;  // NVFP4 weights (W4A4 or W4A16)
    constexpr bool BW = FM == kFmtBF;                    // bf16 weights (no scales)
    constexpr bool BF = FM != kFmtNV;                    // bf16 operands and MFMA
    constexpr bool A16 = FM == kFmtA16;
    constexpr bool O16 = FM == kFmtA16 || FM == kFmtBF;  // bf16 intermediate out of gate_up
    using Frag = typename std::conditional<BF, bf16x8, half8>::type;
    constexpr int BN = 128 * NS;              // weight rows per workgroup (one N-block)
    constexpr int CV = NV ? 1 : (BW ? 4 : 2);  // 16-byte code loads per weight row per lane per chunk
    static_assert(NS % 2 == 0, "gate_up pairs subtiles");
    __shared__ __attribute__((aligned(16))) uint8_t smem[tile_smem_bytes<FM, GATE_UP, NS, BM>()];

    const int K = p.K, N = p.N, F = N / 2;
    const int NB = GATE_UP ? F / (BN / 2) : N / BN;

    // ---- work item of this workgroup (XCD-contiguous ranges; see the header)
    const int n_tiles = p.ctrl->n_tiles;
    const int per_xcd = (n_tiles * NB + 7) / 8;
    const int b = blockIdx.x;
    if ((b >> 3) >= per_xcd) return;
    int tile, nb;
    if (!expert_major_item<kGroup>((b & 7) * per_xcd + (b >> 3), NB, kBM, n_tiles, p.tile_expert, p.tile_row0, p.offsets,
                           tile, nb))
        return;

    const int el = p.tile_expert[tile];
    const int p0 = p.tile_row0[tile];
    const int rows = min(kBM, p.offsets[el + 1] - p0);
    const int e = p.e_begin + el;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g2 = lane >> 5;
    // packed tile layout (layout.h): per chunk, a lane's 32 codes sit in the chunk's block
    // of its row group at byte (row % 32) * CB + CB/2 * g (NVFP4), in quarters 2g and 2g + 1
    // at 16 (row % 32) (MXFP8: each load of a half-wave one contiguous 512 bytes), or in
    // half g at 64 (row % 32) (bf16); its scales in the block's 4-byte (NVFP4) or 2-byte
    // (MXFP8) row slot
    constexpr int CB = BW ? 128 : layout::code_bytes_per_row(NV);
    constexpr int CBLK = 32 * CB, SBLK = layout::scale_block_bytes(NV);
    constexpr int WSTEP = BW ? 16 : 512;  // bytes between a lane's 16-byte loads of one chunk
    const int64_t kb = K / 64;  // blocks per row group
    const uint8_t *w_codes_e = p.w_codes + (int64_t)e * N * (NV ? K / 2 : (BW ? 2 * K : K));
    const uint8_t *w_scales_e = p.w_scales + (int64_t)e * N * (NV ? K / 16 : K / 32);

    // ---- activation staging: global -> registers -> LDS. Rows past the tile's end load
    // the tile's first row instead of zeros: their accumulators are never stored, and
    // unconditional loads from one global base keep the wait counts per chunk.
    const uint8_t *a_base = static_cast<const uint8_t *>(p.a_vals);
    int64_t a_off[kAItems];
    int a_dst[kAItems];
#pragma unroll
    for (int i = 0; i < kAItems; ++i) {
        const int item = tid + i * kThreads;
        const int r = item >> 3, q = item & 7;
        a_dst[i] = r * kAStride + 16 * q;
        const int pos = p0 + (r < rows ? r : 0);
        const int64_t arow = p.gather_by_token ? p.sorted_slot[pos] / p.top_k : pos;
        a_off[i] = arow * K * 2 + 16 * q;
    }
    const float scl = FM == kFmtNV ? p.a_tscale[0] * p.w_tscale[e] : (A16 ? p.w_tscale[e] : 1.0f);

    // software pipeline: activations two chunks ahead in two register sets (chunk c + 2
    // is loaded while chunk c is multiplied, and stored to LDS at the end of chunk c + 1),
    // weights WR chunks ahead in a WR-slot register ring
    constexpr int WR = MOE_TILE_WR;
    const int n_chunks = K / kKC;  // a multiple of WR (see tile_gemm_supported)

#define MOE_LOAD_A(set, c)                                                                                 \
    _Pragma("unroll") for (int i = 0; i < AI; ++i) a_reg[set][i] =                                        \
        *reinterpret_cast<const u32x4 *>(a_base + a_off[i] + 2 * kKC * (c));
#define MOE_STORE_A(buf, set)                                                                              \
    _Pragma("unroll") for (int i = 0; i < AI; ++i)                                                         \
        *reinterpret_cast<u32x4 *>(smem + (buf) * kAStage + a_dst[i]) = a_reg[set][i];
#define MOE_LOAD_W(slot, c)                                                                                \
    _Pragma("unroll") for (int ns = 0; ns < NS; ++ns) {                                                    \
        _Pragma("unroll") for (int v = 0; v < CV; ++v) wcode[slot][ns][v] =                                \
            *reinterpret_cast<const u32x4 *>(wc[ns] + (int64_t)CBLK * (c) + WSTEP * v);                    \
        wsc[slot][ns] = BW ? 0u : *reinterpret_cast<const uint32_t *>(ws[ns] + (int64_t)SBLK * (c));      \
    }

    // The tile for its first MSA 32-row M-subtiles (rows 0 .. 32 MSA - 1) and the NS
    // 32-row weight subtiles of each wave; gate_up pairs gate subtile q with up subtile
    // q + NS / 2.
    auto run = [&](auto msa_c) __attribute__((always_inline)) {
        constexpr int MSA = decltype(msa_c)::value;
        constexpr int AI = kAItems * MSA / kMS;  // activation loads per thread per chunk

        // ---- this lane's weight rows, one per N subtile (each subtile is one row group)
        const uint8_t *wc[NS];
        const uint8_t *ws[NS];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            int row;
            if (GATE_UP) {
                const int col = nb * (BN / 2) + wave * 16 * NS + 32 * (ns % (NS / 2)) + l32;
                row = ns < NS / 2 ? col : F + col;
            } else {
                row = nb * BN + wave * 32 * NS + 32 * ns + l32;
            }
            const int64_t blk0 = (int64_t)(row >> 5) * kb;
            wc[ns] = w_codes_e + blk0 * CBLK +
                     (BW ? 2048 * g2 + 64 * l32 : (NV ? l32 * CB + (CB / 2) * g2 : 1024 * g2 + 16 * l32));
            ws[ns] = BW ? nullptr : w_scales_e + blk0 * SBLK + (NV ? 4 * l32 : 4 * (l32 >> 1));
        }

        float16_t acc[MSA][NS];
#pragma unroll
        for (int i = 0; i < MSA; ++i)
#pragma unroll
            for (int j = 0; j < NS; ++j) acc[i][j] = (float16_t){};

        u32x4 a_reg[2][AI];
        u32x4 wcode[WR][NS][CV];
        uint32_t wsc[WR][NS];
        MOE_LOAD_A(0, 0);
        MOE_STORE_A(0, 0);
        MOE_LOAD_A(1, 1);
#pragma unroll
        for (int r = 0; r < WR; ++r) { MOE_LOAD_W(r, r); }
        __syncthreads();

        for (int c0 = 0; c0 < n_chunks; c0 += WR) {
#pragma unroll
            for (int j = 0; j < WR; ++j) {
                const int c = c0 + j;
                // LDS buffer c%2 holds chunk c, register set (c+1)%2 chunk c + 1, weight slot
                // j chunk c. Prefetches past the end reload chunk n - 1 (in bounds, unused),
                // so the body has no branches and every wait count is exact.
                MOE_LOAD_A(j & 1, min(c + 2, n_chunks - 1));
                __builtin_amdgcn_sched_barrier(0);
                const uint8_t *abuf = smem + (j & 1) * kAStage;
                // scale words: NVFP4 holds the row's 4 block scales of the chunk (this lane's
                // pair is bytes 2g, 2g+1); MXFP8 holds two rows' 2 block scales (this lane's
                // is byte 2 (row % 2) + g)
                half2_t sc_nv[NS];
                float sc_mx[NS];
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) {
                    if constexpr (NV) {
                        sc_nv[ns] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wsc[j][ns] >> (16 * g2), 1.0f, false);
                    } else if constexpr (!BW) {
                        sc_mx[ns] = __uint_as_float(((wsc[j][ns] >> (8 * (2 * (l32 & 1) + g2))) & 0xffu) << 23);
                    }
                }
#pragma unroll
                for (int s = 0; s < kKC / 16; ++s) {
                    Frag af[MSA];
#pragma unroll
                    for (int ms = 0; ms < MSA; ++ms)
                        af[ms] = *reinterpret_cast<const Frag *>(abuf + (32 * ms + l32) * kAStride + 64 * g2 + 16 * s);
#pragma unroll
                    for (int ns = 0; ns < NS; ++ns) {
                        if constexpr (NV) {
                            if constexpr (A16) {
                                const bf16x8 bf = dequant_nvfp4_bf16(wcode[j][ns][0][s], (float)sc_nv[ns][s >> 1]);
#pragma unroll
                                for (int ms = 0; ms < MSA; ++ms)
                                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                            } else {
                                const _Float16 sc = sc_nv[ns][s >> 1];
                                const half8 bf = dequant_nvfp4(wcode[j][ns][0][s], sc);
#pragma unroll
                                for (int ms = 0; ms < MSA; ++ms)
                                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                            }
                        } else if constexpr (BW) {
                            const bf16x8 bf = __builtin_bit_cast(bf16x8, wcode[j][ns][s]);  // the stored values
#pragma unroll
                            for (int ms = 0; ms < MSA; ++ms)
                                acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                        } else {
                            const u32x4 q = wcode[j][ns][s >> 1];
                            const u32x2 cw = (s & 1) ? (u32x2){q.z, q.w} : (u32x2){q.x, q.y};
                            const bf16x8 bf = dequant_mxfp8(cw, sc_mx[ns]);
#pragma unroll
                            for (int ms = 0; ms < MSA; ++ms)
                                acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bf, acc[ms][ns], 0, 0, 0);
                        }
                    }
                }
                MOE_LOAD_W(j, min(c + WR, n_chunks - 1));
                // buffer (c+1)%2 was last read in chunk c - 1, before the previous barrier
                MOE_STORE_A((j + 1) & 1, (j + 1) & 1);
                __syncthreads();
            }
        }

        // ---- epilogue: accumulator v of lane l = row 32 ms + 8(v/4) + 4 g2 + v%4, column l32
        // Outputs leave 32 x 32 at a time through this wave's LDS tile (the A stages are
        // free: every wave passed the loop's last barrier), each lane storing 16-byte row
        // pieces instead of one 2- or 4-byte store per accumulator element (the store
        // instructions were a measurable share of the prefill epilogues). Rows past the
        // tile's end are not stored.
        float *yt = reinterpret_cast<float *>(smem) + wave * 32 * kYStride;
        auto stage = [&](const float (&val)[16]) __attribute__((always_inline)) {
            __builtin_amdgcn_wave_barrier();  // the previous tile's reads of yt come first
#pragma unroll
            for (int v = 0; v < 16; ++v) yt[(8 * (v / 4) + 4 * g2 + (v % 4)) * kYStride + l32] = val[v];
            __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave complete in issue order
        };
        // fp32 rows: lane (r = lane / 8 + 8 j, piece lane % 8) of the staged tile
        auto put_f32 = [&](int ms, float *out, int64_t ld, int col0, bool nt) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = (lane >> 3) + 8 * j, q = lane & 7, m = 32 * ms + r;
                const float4 x = *reinterpret_cast<const float4 *>(yt + r * kYStride + 4 * q);
                if (m < rows) store_f4(out + (int64_t)(p0 + m) * ld + col0 + 4 * q, x, nt);
            }
        };
        if (GATE_UP && O16) {
            // W4A16 and bf16 experts: the SwiGLU output rounded to bf16 (nearest even) is
            // the down GEMM's input; lane (r = lane / 4 + 16 j, eighth lane % 4) stores 8
            // values
#pragma unroll
            for (int q = 0; q < NS / 2; ++q) {
                const int f0 = nb * (BN / 2) + wave * 16 * NS + 32 * q;
#pragma unroll
                for (int ms = 0; ms < MSA; ++ms) {
                    float val[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) val[v] = swiglu(acc[ms][q][v] * scl, acc[ms][q + NS / 2][v] * scl);
                    stage(val);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int r = (lane >> 2) + 16 * j, e8 = lane & 3, m = 32 * ms + r;
                        const float4 x0 = *reinterpret_cast<const float4 *>(yt + r * kYStride + 8 * e8);
                        const float4 x1 = *reinterpret_cast<const float4 *>(yt + r * kYStride + 8 * e8 + 4);
                        if (m < rows) {
                            const int64_t o = (int64_t)(p0 + m) * F + f0 + 8 * e8;
                            const __bf16 b[8] = {(__bf16)x0.x, (__bf16)x0.y, (__bf16)x0.z, (__bf16)x0.w,
                                                 (__bf16)x1.x, (__bf16)x1.y, (__bf16)x1.z, (__bf16)x1.w};
                            *reinterpret_cast<u32x4 *>(static_cast<__bf16 *>(p.o_vals) + o) = __builtin_bit_cast(u32x4, b);
                            if (p.o_tap) {
                                store_f4(p.o_tap + o, x0, false);
                                store_f4(p.o_tap + o + 4, x1, false);
                            }
                        }
                    }
                }
            }
        } else if (GATE_UP && NV) {
            uint32_t amax = 0;
#pragma unroll
            for (int q = 0; q < NS / 2; ++q) {
                const int f0 = nb * (BN / 2) + wave * 16 * NS + 32 * q;
#pragma unroll
                for (int ms = 0; ms < MSA; ++ms) {
                    float val[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                        const float hv = swiglu(acc[ms][q][v] * scl, acc[ms][q + NS / 2][v] * scl);
                        val[v] = hv;
                        if (m < rows) amax = max(amax, __float_as_uint(hv) & 0x7fffffffu);
                    }
                    stage(val);
                    put_f32(ms, p.out_f32, F, f0, false);
                }
            }
            for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
            if (lane == 0 && amax) atomic_max_grow(p.amax_bits, amax);
        } else if (GATE_UP) {
            // MXFP8: the wave's SwiGLU tile (32 MSA rows x 16 NS columns, 32-column
            // blocks) goes through its own LDS region; lane r then quantises whole blocks
            // of row r with 16-byte stores. The A stages are free: every wave passed the
            // loop's last barrier.
            float *epi = reinterpret_cast<float *>(smem) + wave * kBM * kEpiStride<NS>();
#pragma unroll
            for (int q = 0; q < NS / 2; ++q)
#pragma unroll
                for (int ms = 0; ms < MSA; ++ms)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                        epi[m * kEpiStride<NS>() + 32 * q + l32] = swiglu(acc[ms][q][v], acc[ms][q + NS / 2][v]);
                    }
            __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave complete in issue order
            for (int m = lane; m < 32 * MSA; m += 64) {
                if (m >= rows) continue;
                const int64_t row = p0 + m;
#pragma unroll
                for (int q = 0; q < NS / 2; ++q) {
                    const int fb = nb * (BN / 2) + wave * 16 * NS + 32 * q;  // first column of the block
                    float x[32];
#pragma unroll
                    for (int i = 0; i < 32; ++i) x[i] = epi[m * kEpiStride<NS>() + 32 * q + i];
                    uint32_t cw[8];
                    const int sc8 = mxfp8_quant_block(x, cw);
                    u32x4 *dst = reinterpret_cast<u32x4 *>(p.o_codes + row * F + fb);
                    dst[0] = (u32x4){cw[0], cw[1], cw[2], cw[3]};
                    dst[1] = (u32x4){cw[4], cw[5], cw[6], cw[7]};
                    p.o_scales[row * (F / 32) + fb / 32] = (uint8_t)sc8;
                    store_dequant_mxfp8_32(static_cast<uint8_t *>(p.o_vals) + (row * F + fb) * 2, cw, sc8);
                    if (p.o_tap) {
                        float4 *t = reinterpret_cast<float4 *>(p.o_tap + row * F + fb);
#pragma unroll
                        for (int i = 0; i < 8; ++i) t[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
                    }
                }
            }
        } else {
            // y, stored non-temporally (store_y: written once, read once by the combine)
#pragma unroll
            for (int ms = 0; ms < MSA; ++ms)
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) {
                    float val[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) val[v] = NV ? acc[ms][ns][v] * scl : acc[ms][ns][v];
                    stage(val);
                    put_f32(ms, p.out_f32, N, nb * BN + wave * 32 * NS + 32 * ns, true);
                }
        }
    };
#undef MOE_LOAD_A
#undef MOE_STORE_A
#undef MOE_LOAD_W

    // A tile runs only as many 32-row M-subtiles as it has rows (an expert's last tile is
    // usually short: at about 170 rows per expert half of the last 64-row tiles hold at
    // most 32 rows).
    constexpr bool SHORT = MOE_TILE_SHORT && (FM != kFmtBF || kMS == 4);  // bf16 64-row: no gain, more spills
    if (SHORT && rows <= 32)
        run(std::integral_constant<int, 1>{});
    else if (kMS == 4 && rows <= 64)
        run(std::integral_constant<int, kMS == 4 ? 2 : kMS>{});
    else
        run(std::integral_constant<int, kMS>{});
}

template <int FM, bool GATE_UP>
hipError_t launch_t(const GemmArgs &a, int32_t max_tiles, hipStream_t s) {
    constexpr int NS = tile_ns<FM>(), BM = tile_bm<FM>();
    constexpr int BN = 128 * NS;
    const int64_t nb = GATE_UP ? (a.N / 2) / (BN / 2) : a.N / BN;
    const int64_t items = (int64_t)max_tiles * nb;
    const int64_t grid = (items + 7) / 8 * 8;
    hipLaunchKernelGGL((tile_gemm_kernel<FM, GATE_UP, NS, BM>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int32_t tile_gemm_bm(int fm) {
    switch (fm) {
        case kFmtNV: return tile_bm<kFmtNV>();
        case kFmtMX8: return tile_bm<kFmtMX8>();
        case kFmtA16: return tile_bm<kFmtA16>();
        case kFmtBF: return tile_bm<kFmtBF>();
        default: return 64;
    }
}

template <int FM>
bool supported_t(int32_t K, int32_t N, bool gate_up) {
    constexpr int BN = 128 * tile_ns<FM>();
    return K > 0 && N > 0 && K % (MOE_TILE_WR * kKC) == 0 && (gate_up ? (N / 2) % (BN / 2) == 0 : N % BN == 0);
}

bool tile_gemm_supported(int fm, int32_t K, int32_t N, bool gate_up) {
    switch (fm) {
        case kFmtNV: return supported_t<kFmtNV>(K, N, gate_up);
        case kFmtMX8: return supported_t<kFmtMX8>(K, N, gate_up);
        case kFmtA16: return supported_t<kFmtA16>(K, N, gate_up);
        case kFmtBF: return supported_t<kFmtBF>(K, N, gate_up);
        default: return false;
    }
}

hipError_t launch_tile_gemm(const GemmArgs &a, int fm, bool gate_up, int32_t max_tiles, hipStream_t s) {
    switch (fm) {
        case kFmtNV: return gate_up ? launch_t<kFmtNV, true>(a, max_tiles, s) : launch_t<kFmtNV, false>(a, max_tiles, s);
        case kFmtMX8: return gate_up ? launch_t<kFmtMX8, true>(a, max_tiles, s) : launch_t<kFmtMX8, false>(a, max_tiles, s);
        case kFmtA16: return gate_up ? launch_t<kFmtA16, true>(a, max_tiles, s) : launch_t<kFmtA16, false>(a, max_tiles, s);
        case kFmtBF: return gate_up ? launch_t<kFmtBF, true>(a, max_tiles, s) : launch_t<kFmtBF, false>(a, max_tiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
