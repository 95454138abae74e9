// gemm_mx.hip - grouped expert GEMMs for the OCP MX formats on the gfx950 scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4: MXFP8 (E4M3 codes with an E8M0 scale per 32 values,
// the layers 40-47 experts of the vLLM recipe "thinkingmachines/Inkling-2-Small",
// section "Overview") and MXFP4 (E2M1 codes, same scales; the AMD variant of the vLLM
// recipe "thinkingmachines/Inkling-Small", section "Variants"), weights and activations
// both in the format.
//
// The instruction takes the codes and E8M0 scales as they are stored: no expansion, no
// tensor scale. Per 64-wide K chunk lane l supplies row (column) l % 32 with the scale
// byte of block l / 32 of that row:
//  - FP4: the 32 values of block l / 32 (16 code bytes, element 2i in the low nibble);
//  - FP8: registers 0-3 take 16 values of the chunk's first 32-block and registers 4-7
//    16 values of the second (measured on gfx950 by tests/test_gpu_fp8_mfma_accuracy.py:
//    the scale byte of lane l applies to block l / 32 of its row, and a lane's registers
//    0-3 belong to the first block whatever l / 32 is). Lane half g takes k = 16g .. +15
//    and 32 + 16g .. +15, two 16-byte pieces.
// In the packed weight layouts (layout.h) a wave's operand of one chunk is then one
// contiguous run: MXFP4 keeps a block's two 32-column halves apart ([2][32 rows][16 B],
// lane l the l-th 16 bytes), MXFP8 its four 16-column quarters ([4][32 rows][16 B]:
// lane half g reads quarters g and 2 + g, each load instruction 1 KiB contiguous); the
// scales are one 64-byte run. The products are exact; the sums are not those of a
// sequential fp32 chain: the same test measures the FP8 sums within about 2e-6 of the
// sum of |products| (the 16-bit route: 2e-8), an error made inside each instruction,
// and FP4 within 1.6e-7 (0 with equal block exponents).
//
//  - workgroup tile 128 sorted rows x 256 weight rows, 4 waves side by side in N, each
//    128 x 64 as 4 x 2 MFMA tiles (each weight operand feeds four MFMAs); a tile runs only
//    the 32-row subtiles that hold rows (an expert's last tile, every tile at decode);
//    gate_up waves pair gate row f with up row F + f;
//  - the activation tile (shared by the four waves) goes through double-buffered LDS in
//    groups of 128 code bytes per row (four FP4 chunks, two FP8 chunks), loaded as whole
//    128-byte pieces of the gathered token rows; each lane loads its weight operands
//    straight from global memory into a register ring; one barrier per group;
//  - the E8M0 scales of the tile's activation rows (K / 32 bytes per row) are staged in LDS
//    once per tile, each load instruction reading consecutive bytes of one or two rows;
//    loaded with each group's codes instead, 2 bytes per row and group, every instruction
//    touched 32 gathered rows' lines, and those loads took about 10% of the MXFP8 and MXFP4
//    prefill gate_up (a timing-only copy without them: skewed-mxfp8 3.30 -> 2.96 ms,
//    prefill-mxfp4-ep4 0.295 -> 0.265 ms). K <= 8192 (the LDS region's size);
//  - work items are ordered expert-major and dealt to the 8 XCDs in contiguous ranges, as
//    in the tile kernels;
//  - gate_up epilogue: SwiGLU in fp32, then each wave's rows x 32 tile goes through LDS and
//    lane r quantises row r's 32-block to the layer's format (16- or 32-byte code store,
//    one scale byte).
// FP8 rows (ROWS; E4M3 with one fp32 scale per activation row and per weight channel, the
// fp8 variant of the vLLM recipe "thinkingmachines/Inkling-Small") runs the FP8 kernel
// with every E8M0 scale operand 127 (2^0) and no scale loads; its epilogues multiply the
// sums by fl32(row scale * channel scale) (the row scales staged in LDS), and gate_up
// writes the fp32 SwiGLU output, whose per-row scale needs the whole row (quant.hip).
// Accumulator v of lane l is row 8(v/4) + 4(l/32) + v%4, column l%32.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

using namespace gemm_detail;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

#ifndef MOE_MX_GROUP
#define MOE_MX_GROUP 4  // M-tiles per expert-major work group of the down GEMM (gemm_common.h)
#endif
constexpr int kBM = 128, kMS = kBM / 32, kThreads = 256, kGroup = MOE_MX_GROUP;
// gate_up takes each expert's M-tiles as one group (a group size above any expert's tile
// count below 2^19 rows; a larger expert still splits into groups, each correct): every
// N-block's weight panel then passes the XCD's L2 once for all of the expert's tiles.
// Measured against groups of 4 (same box): skewed-mxfp8 gate_up 3.35 -> 3.25 ms,
// prefill-mxfp4-ep4 0.294 -> 0.290 ms; groups of 16, 32 and 64 fell in between. The
// down GEMM keeps groups of 4: groups of 2 and 8 were slower there (1.85 -> 1.88, 1.89 ms).
constexpr int kGroupGateUp = 4096;
constexpr int kARow = 144;                     // LDS bytes per A row: 128 of codes + 16 (bank spread)
constexpr int kACodes = kBM * kARow;           // one A buffer: [kBM rows][kARow]
constexpr int kMaxK = 8192;                    // longest K of the staged row scales
constexpr int kAScales = kBM * (kMaxK / 32 + 8);  // [kBM rows][K / 32 + 8] after the two A buffers
constexpr int kEpiStride = 33;  // floats per row of a wave's SwiGLU tile (bank spread)
constexpr int kYStride = 40;    // floats per row of a wave's 32 x 32 y tile (16-byte rows; lanes 32-63
                                // write 4 rows down, 32 banks away)

#ifndef MOE_MX4_RING
#define MOE_MX4_RING 4
#endif
#ifndef MOE_MX8_RING
#define MOE_MX8_RING 2  // FP8 operands are twice as wide: a deeper ring spills at two waves per SIMD
#endif
#ifndef MOE_MX4_NS
#define MOE_MX4_NS 2
#endif
#ifndef MOE_MX8_NS
#define MOE_MX8_NS 2
#endif
#ifndef MOE_MX8_WAVES
#define MOE_MX8_WAVES 2
#endif

// per-format constants: code bytes per row per 64-wide chunk, chunks per A group (128
// code bytes per row), weight ring depth in chunks, bytes of one 32 x 64 weight block,
// 32-row weight subtiles per wave (NS; a workgroup covers 128 NS weight rows) and the
// waves per SIMD the register budget is set for
template <bool FP8>
struct Mx {
    static constexpr int CB = FP8 ? 64 : 32;
    static constexpr int kGrp = 128 / CB;
    static constexpr int kRing = FP8 ? MOE_MX8_RING : MOE_MX4_RING;
    static constexpr int kCodeBlock = 32 * CB, kScaleBlock = 64;
    static constexpr int kFmt = FP8 ? 0 : 4;  // cbsz / blgp: E4M3 or E2M1 operands
    static constexpr int NS = FP8 ? MOE_MX8_NS : MOE_MX4_NS;
    static constexpr int kBN = 128 * NS;
    static constexpr int kWaves = FP8 ? MOE_MX8_WAVES : 2;
    static_assert(kRing % kGrp == 0, "the B ring turns over whole A groups");
    static_assert(NS % 2 == 0, "gate_up pairs subtiles");
};

// four consecutive y values of a row, stored non-temporally like store_y (16-byte aligned)
__device__ __forceinline__ void store_y4(float *p, float4 v) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((f4v){v.x, v.y, v.z, v.w}, reinterpret_cast<f4v *>(p));
}

__device__ __forceinline__ v8i operand(u32x4 lo, u32x4 hi) {
    return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// NT: the weight code loads are marked non-temporal. At decode each (expert, weight row)
// panel is read by a single M-tile, and a wave's load covers whole lines.
template <bool FP8, bool ROWS, bool GATE_UP, bool NT>
__global__ void __launch_bounds__(kThreads, (Mx<FP8>::kWaves)) mx_gemm_kernel(const GemmArgs p) {
    static_assert(FP8 || !ROWS, "row scales come with E4M3 codes");
    using X = Mx<FP8>;
    constexpr int kGrp = X::kGrp, kRing = X::kRing, kCodeBlock = X::kCodeBlock, kScaleBlock = X::kScaleBlock;
    constexpr int kNS = X::NS, kBN = X::kBN;
    constexpr int kLoop = 2 * kACodes + (ROWS ? 0 : kAScales);  // A tiles and row scales
    constexpr int kEpi = GATE_UP && !ROWS ? 4 * kBM * kEpiStride * 4 : 0;  // SwiGLU tiles
    constexpr int kLds = kEpi > kLoop ? kEpi : kLoop;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];  // A tiles and scales; then the SwiGLU tiles

    const int K = p.K, N = p.N, F = N / 2;
    const int NB = GATE_UP ? F / (kBN / 2) : N / kBN;

    // ---- work item of this workgroup (XCD-contiguous ranges, as in the tile kernels)
    const int n_tiles = p.ctrl->n_tiles;
    const int per_xcd = (n_tiles * NB + 7) / 8;
    const int b = blockIdx.x;
    if ((b >> 3) >= per_xcd) return;
    int tile, nb;
    if (!expert_major_item<(GATE_UP ? kGroupGateUp : kGroup)>((b & 7) * per_xcd + (b >> 3), NB, kBM, n_tiles,
                                                              p.tile_expert, p.tile_row0, p.offsets, tile, nb))
        return;

    const int el = p.tile_expert[tile];
    const int p0 = p.tile_row0[tile];
    const int rows = min(kBM, p.offsets[el + 1] - p0);
    const int e = p.e_begin + el;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, g2 = lane >> 5;
    const int64_t kb = K / 64;                  // 64-wide blocks per weight row group
    const int64_t row_bytes = FP8 ? K : K / 2;  // code bytes of one activation or weight row
    const uint8_t *wc_e = p.w_codes + (int64_t)e * N * row_bytes;
    const uint8_t *ws_e = ROWS ? nullptr : p.w_scales + (int64_t)e * N * (K / 32);

    // Weight scales: a chunk's scale block of a row group is 64 bytes (byte o = 2 row + g
    // for MXFP8, 32 g + row for MXFP4) and a row group's blocks are consecutive over the
    // chunks. SDW (MXFP8 outside decode): the wave's kNS groups of one ring turn (kRing
    // chunks) are kNS runs of 64 kRing bytes, loaded as SW dwords per lane (dword D = 64 h
    // + lane is dword D % 16 of chunk (D / 16) % kRing of subtile D / (16 kRing)), and each
    // chunk's MFMAs take the lane's byte from the lane holding it (ds_bpermute, then a
    // shift: the instruction reads the low byte). Otherwise each lane loads its byte per
    // subtile and chunk. Measured (bench hipEvents, one box): skewed-mxfp8 gate_up 2.99 ->
    // 2.90 ms and down 1.83 -> 1.78 ms with the dwords; prefill-mxfp4-ep4 unchanged, and
    // decode-mxfp8 1.196 -> 1.205 ms (at one 32-row subtile per tile the exchange sits on
    // each chunk's short path), so those keep the byte loads.
    constexpr bool SDW = FP8 && !ROWS && !NT;
    // ---- this lane's B operand rows (weights): the first of its (one or two) 16-byte
    // pieces of a chunk (MXFP4: half g2 at 512 g2; MXFP8: quarters g2 and 2 + g2 at 512 g2
    // and 512 g2 + 1024), and its scale byte (SDW: the scale blocks of the wave's row
    // groups, uniform)
    const uint8_t *bc[kNS];
    const uint8_t *bs[kNS];
#pragma unroll
    for (int ns = 0; ns < kNS; ++ns) {
        int row;
        if (GATE_UP) {
            const int col = nb * (kBN / 2) + wave * 16 * kNS + 32 * (ns % (kNS / 2)) + l32;
            row = ns < kNS / 2 ? col : F + col;
        } else {
            row = nb * kBN + wave * 32 * kNS + 32 * ns + l32;
        }
        const int64_t blk0 = (int64_t)(row >> 5) * kb;
        bc[ns] = wc_e + blk0 * kCodeBlock + g2 * 512 + (row & 31) * 16;
        bs[ns] = ROWS ? nullptr
                      : ws_e + blk0 * kScaleBlock + (SDW ? 0 : (FP8 ? 2 * (row & 31) + g2 : g2 * 32 + (row & 31)));
    }
    constexpr int SW = SDW ? kRing * kNS / 4 : 1;  // scale dwords per lane per ring turn
    static_assert(!SDW || (16 * kRing * kNS) % 64 == 0, "whole dwords per lane");
    const uint8_t *s_src[SW];
    int s_cj[SW];
#pragma unroll
    for (int h = 0; h < SW; ++h) {
        const int D = 64 * h + lane, ns = D / (16 * kRing);
        const uint8_t *base = bs[0];
#pragma unroll
        for (int n = 1; n < kNS; ++n)
            if (ns == n) base = bs[n];
        s_src[h] = SDW ? base + 4 * (D % 16) : nullptr;
        s_cj[h] = (D / 16) % kRing;
    }
    const int s_o = FP8 ? 2 * l32 + g2 : 32 * g2 + l32;  // this lane's byte in a scale block
    const int s_perm = 4 * (s_o / 4), s_shift = 8 * (s_o % 4);
    const int n_chunks = K / 64;
    const int n_groups = (n_chunks + kGrp - 1) / kGrp;
    auto a_row = [&](int r) -> int64_t {
        const int pos = p0 + (r < rows ? r : 0);
        return p.gather_by_token ? p.sorted_slot[pos] / p.top_k : pos;
    };

    // The tile for its first MSA 32-row M-subtiles (rows 0 .. 32 MSA - 1): an expert's last
    // tile (and every tile at decode) usually holds fewer than kBM rows, and its loop only
    // loads and multiplies the subtiles holding rows.
    auto run = [&](auto msa_c) __attribute__((always_inline)) {
        constexpr int MSA = decltype(msa_c)::value;
        constexpr int AQ = MSA;                   // 16-byte A pieces per thread per group (32 rows each)
        // ---- B operand ring: chunk c + kRing - 1 is loaded into slot (c - 1) % kRing while
        // chunk c is multiplied; loads past the end repeat the last chunk (in bounds, unused)
        u32x4 breg[kRing][kNS][FP8 ? 2 : 1];
        int bsc[kRing][kNS];
        auto b_load = [&](int slot, int c) {
#pragma unroll
            for (int ns = 0; ns < kNS; ++ns) {
#pragma unroll
                for (int h = 0; h < (FP8 ? 2 : 1); ++h) {
                    const u32x4 *src = reinterpret_cast<const u32x4 *>(bc[ns] + (int64_t)kCodeBlock * c + 1024 * h);
                    if constexpr (NT)
                        breg[slot][ns][h] = __builtin_nontemporal_load(src);
                    else
                        breg[slot][ns][h] = *src;
                }
                if constexpr (!SDW) bsc[slot][ns] = ROWS ? 127 : bs[ns][(int64_t)kScaleBlock * c];
            }
        };
        // the weight scales of the ring turn starting at chunk c0 (chunks past the end
        // reread the last, in bounds and unused); sd_cur holds the current turn's
        uint32_t sd_cur[SW], sd_next[SW];
        auto s_load = [&](uint32_t(&dst)[SW], int c0) {
            if constexpr (SDW) {
#pragma unroll
                for (int h = 0; h < SW; ++h)
                    dst[h] = *reinterpret_cast<const uint32_t *>(s_src[h] +
                                                               (int64_t)kScaleBlock * min(c0 + s_cj[h], n_chunks - 1));
            }
        };
        // scale operand of subtile ns for chunk `slot` of the current turn
        auto b_scale = [&](int slot, int ns) -> int {
            if constexpr (!SDW) return bsc[slot][ns];
            const int q = 16 * (slot + kRing * ns);
            return __builtin_amdgcn_ds_bpermute(4 * (q % 64) + s_perm, (int)sd_cur[q / 64]) >> s_shift;
        };
        // ---- A tile (activations) through LDS, one group (128 code bytes per row) at a
        // time, double-buffered. Thread t loads 16-byte pieces i = t + 256 q (row i / 8,
        // piece i % 8: a wave covers 8 whole 128-byte pieces of rows, so the gathered token
        // rows are read line by line). Rows past the tile's end read the tile's first row
        // (in bounds; never stored); pieces past the end of K reread the group's first
        // (unused).
        // The tile's activation row scales go to LDS once: wave w takes rows w + 4 j, lane l
        // dword l of the row's K / 32 bytes (K <= kMaxK: at most 64 dwords), into LDS rows
        // of srow bytes, stored after the first A group's loads are issued and read per
        // group by a_scales; lane j looks up row w + 4 j and each row's loads take that
        // with readlane.
        // The row lookups (sorted slots, in bounds for both GEMMs) are loaded without a
        // branch and the first weight chunks after them, so one wait covers every lookup
        // while the weights are in flight (a lookup per row under a branch made the
        // compiler wait for each in turn before anything else was issued).
        const int piece = threadIdx.x & 7;
        constexpr int SQ = ROWS ? 1 : 8 * MSA;    // rows per wave
        const int sdw = K / 128;                  // scale dwords per row (K % 128 == 0)
        const int srow = K / 32 + 8;              // LDS bytes per row: 8-byte aligned, rows spread over banks
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        int pos[AQ + 1], slot_of[AQ + 1];
#pragma unroll
        for (int q = 0; q <= AQ; ++q) {
            const int r = q < AQ ? 32 * q + (threadIdx.x >> 3) : wave_u + 4 * min(lane, SQ - 1);
            pos[q] = p0 + (r < rows ? r : 0);
            slot_of[q] = p.sorted_slot[pos[q]];
        }
#pragma unroll
        for (int r = 0; r < kRing - 1; ++r) b_load(r, min(r, n_chunks - 1));
        s_load(sd_cur, 0);
        // an (empty) use of every lookup here: the compiler would otherwise move a lookup
        // into the branch on gather_by_token, behind the weight loads, and wait for all
#pragma unroll
        for (int q = 0; q <= AQ; ++q) asm volatile("" ::"v"(slot_of[q]));
        const uint8_t *ap[AQ];
#pragma unroll
        for (int q = 0; q < AQ; ++q)
            ap[q] = p.a_codes + (int64_t)(p.gather_by_token ? slot_of[q] / p.top_k : pos[q]) * row_bytes;
        uint32_t s_pre[SQ];
        if constexpr (!ROWS) {
            const int tok_l = p.gather_by_token ? slot_of[AQ] / p.top_k : pos[AQ];
#pragma unroll
            for (int j = 0; j < SQ; ++j) {
                const uint8_t *src = p.a_scales + (int64_t)__builtin_amdgcn_readlane(tok_l, j) * (K / 32);
                if (lane < sdw) s_pre[j] = reinterpret_cast<const uint32_t *>(src)[lane];
            }
        }
        auto s_store = [&]() {
            if constexpr (!ROWS) {
#pragma unroll
                for (int j = 0; j < SQ; ++j)
                    if (lane < sdw)
                        reinterpret_cast<uint32_t *>(lds + 2 * kACodes + (wave_u + 4 * j) * srow)[lane] = s_pre[j];
            }
        };
        u32x4 a_pf[AQ];
        auto a_load = [&](int g) {
            g = min(g, n_groups - 1);
            const int off = 128 * g + 16 * piece;
            const int off_ok = off < row_bytes ? off : 128 * g;
#pragma unroll
            for (int q = 0; q < AQ; ++q) a_pf[q] = *reinterpret_cast<const u32x4 *>(ap[q] + off_ok);
        };
        auto a_store = [&](int buf) {
            uint8_t *ab = lds + buf * kACodes;
#pragma unroll
            for (int q = 0; q < AQ; ++q)
                *reinterpret_cast<u32x4 *>(ab + (32 * q + (threadIdx.x >> 3)) * kARow + 16 * piece) = a_pf[q];
        };

        float16_t acc[MSA][kNS];
#pragma unroll
        for (int i = 0; i < MSA; ++i)
#pragma unroll
            for (int j = 0; j < kNS; ++j) acc[i][j] = (float16_t){};
        // group g's scale bytes of this lane's rows: byte 2 j + g2 of the group's 2 kGrp
        // (chunk j, block g2), taken by mma as (a_sc[ms][j / 2] >> 16 (j % 2)) & 0xff
        uint32_t a_sc[MSA][2];
        auto a_scales = [&](int g) {
            if constexpr (ROWS) return;
            const uint8_t *sb = lds + 2 * kACodes + 2 * kGrp * g;
#pragma unroll
            for (int ms = 0; ms < MSA; ++ms) {
                const uint8_t *sr = sb + (32 * ms + l32) * srow;
                if constexpr (kGrp == 4) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(sr);
                    a_sc[ms][0] = v.x >> (8 * g2);
                    a_sc[ms][1] = v.y >> (8 * g2);
                } else {
                    a_sc[ms][0] = *reinterpret_cast<const uint32_t *>(sr) >> (8 * g2);
                    a_sc[ms][1] = 0;
                }
            }
        };
        // chunk j of the group in LDS buffer buf times the B operands in ring slot `slot`
        auto mma = [&](int buf, int j, int slot) {
            const uint8_t *ab = lds + buf * kACodes;
            v8i af[MSA];
#pragma unroll
            for (int ms = 0; ms < MSA; ++ms) {
                const uint8_t *ar = ab + (32 * ms + l32) * kARow + X::CB * j + 16 * g2;
                const u32x4 lo = *reinterpret_cast<const u32x4 *>(ar);
                if constexpr (FP8)
                    af[ms] = operand(lo, *reinterpret_cast<const u32x4 *>(ar + 32));
                else
                    af[ms] = operand(lo, (u32x4){});
            }
            int sb[kNS];
#pragma unroll
            for (int ns = 0; ns < kNS; ++ns) sb[ns] = b_scale(slot, ns);
#pragma unroll
            for (int ms = 0; ms < MSA; ++ms) {
                // scale byte of chunk j, block g2: byte 2 j + g2 of the row's scales
                const int sa = ROWS ? 127 : (int)((a_sc[ms][j >> 1] >> (16 * (j & 1))) & 0xffu);
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns) {
                    v8i bf;
                    if constexpr (FP8)
                        bf = operand(breg[slot][ns][0], breg[slot][ns][FP8 ? 1 : 0]);
                    else
                        bf = operand(breg[slot][ns][0], (u32x4){});
                    acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[ms], bf, acc[ms][ns], X::kFmt, X::kFmt, 0, sa, 0, sb[ns]);
                }
            }
        };
        // after the last chunk of group g: group g + 1 into the other buffer (last read in
        // group g - 1, before the previous barrier), group g + 2 into registers
        auto next_group = [&](int g) {
            a_store((g & 1) ^ 1);
            a_load(g + 2);
            __syncthreads();
        };

        a_load(0);
        s_store();
        a_store(0);
        a_load(1);
        __syncthreads();
        // whole ring turns without a branch inside (a conditional use would let the
        // compiler sink the prefetches into it), then the last n_chunks % kRing chunks,
        // already loaded
        const int n_full = n_chunks - n_chunks % kRing;
        for (int c0 = 0; c0 < n_full; c0 += kRing) {
#pragma unroll
            for (int gi = 0; gi < kRing / kGrp; ++gi) {
                const int g = c0 / kGrp + gi;
                a_scales(g);
#pragma unroll
                for (int j = 0; j < kGrp; ++j) {
                    // keep each chunk's prefetch in place: left alone, the scheduler gathers
                    // the ring's loads at the end of the group and waits for them all at once
                    __builtin_amdgcn_sched_barrier(0);
                    const int slot = gi * kGrp + j;
                    b_load((slot + kRing - 1) % kRing, min(c0 + slot + kRing - 1, n_chunks - 1));
                    if (slot == 0) s_load(sd_next, c0 + kRing);
                    mma(g & 1, j, slot);
                }
                __builtin_amdgcn_sched_barrier(0);
                next_group(g);
            }
            if constexpr (SDW) {
#pragma unroll
                for (int h = 0; h < SW; ++h) sd_cur[h] = sd_next[h];
            }
        }
#pragma unroll
        for (int t = 0; t < kRing - 1; ++t) {
            const int c = n_full + t;
            if (c >= n_chunks) break;
            const int g = c / kGrp;
            if (t % kGrp == 0) a_scales(g);
            mma(g & 1, t % kGrp, t);
            if (t % kGrp == kGrp - 1 && c + 1 < n_chunks) next_group(g);
        }

        // ---- epilogue: accumulator v of lane l = row 32 ms + 8(v/4) + 4 g2 + v%4, column l32
        // A down tile's y goes out 32 x 32 at a time through this wave's LDS tile (after the
        // A buffers are done with): each lane stores 16-byte row pieces, a quarter of the
        // store instructions of one 4-byte store per accumulator (which measured 11% of the
        // skewed-mxfp8 down GEMM and 21% of the prefill-mxfp4-ep4 one in a timing-only copy
        // without y stores). Rows past the tile's end are not stored.
        auto store_y_tile = [&](float *yt, int ms, const float (&val)[16], float *out_col0) __attribute__((always_inline)) {
            __builtin_amdgcn_wave_barrier();  // the previous tile's reads of yt come first
#pragma unroll
            for (int v = 0; v < 16; ++v) yt[(8 * (v / 4) + 4 * g2 + (v % 4)) * kYStride + l32] = val[v];
            __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave complete in issue order
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = (lane >> 3) + 8 * j, q = lane & 7, m = 32 * ms + r;
                const float4 x = *reinterpret_cast<const float4 *>(yt + r * kYStride + 4 * q);
                if (m < rows) store_y4(out_col0 + (int64_t)(p0 + m) * N + 4 * q, x);
            }
        };
        if constexpr (ROWS) {
            // the tile's row scales through LDS (the A tiles are done with)
            __syncthreads();
            float *rs = reinterpret_cast<float *>(lds);
            if (threadIdx.x < 32 * MSA) rs[threadIdx.x] = p.a_rscale[a_row(threadIdx.x)];
            __syncthreads();
            const float *ch = p.w_tscale + (int64_t)e * N;
            if (GATE_UP) {
#pragma unroll
                for (int q = 0; q < kNS / 2; ++q) {
                    const int col = nb * (kBN / 2) + wave * 16 * kNS + 32 * q + l32;
                    const float cg = ch[col], cu = ch[F + col];
#pragma unroll
                    for (int ms = 0; ms < MSA; ++ms)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                            if (m < rows) {
                                const float sr = rs[m];
                                const float g = acc[ms][q][v] * (sr * cg), u = acc[ms][q + kNS / 2][v] * (sr * cu);
                                p.out_f32[(int64_t)(p0 + m) * F + col] = swiglu(g, u);
                            }
                        }
                }
            } else {
                float *yt = reinterpret_cast<float *>(lds) + kBM + wave * 32 * kYStride;  // after the row scales
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns) {
                    const int n0 = nb * kBN + wave * 32 * kNS + 32 * ns;
                    const float cn = ch[n0 + l32];
#pragma unroll
                    for (int ms = 0; ms < MSA; ++ms) {
                        float val[16];
#pragma unroll
                        for (int v = 0; v < 16; ++v) val[v] = acc[ms][ns][v] * (rs[32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4)] * cn);
                        store_y_tile(yt, ms, val, p.out_f32 + n0);
                    }
                }
            }
        } else if (GATE_UP) {
            __syncthreads();  // the SwiGLU tiles reuse the A tiles' LDS
            float *we = reinterpret_cast<float *>(lds) + wave * kBM * kEpiStride;
#pragma unroll
            for (int q = 0; q < kNS / 2; ++q) {  // one 32-column block of the wave per pass
                if (q) __builtin_amdgcn_wave_barrier();  // the previous block's reads first
#pragma unroll
                for (int ms = 0; ms < MSA; ++ms)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int m = 32 * ms + 8 * (v / 4) + 4 * g2 + (v % 4);
                        we[m * kEpiStride + l32] = swiglu(acc[ms][q][v], acc[ms][q + kNS / 2][v]);
                    }
                __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave complete in issue order
                const int fb = nb * (kBN / 2) + wave * 16 * kNS + 32 * q;  // first column of the block
#pragma unroll
                for (int m0 = 0; m0 < 32 * MSA; m0 += 64) {
                    const int m = m0 + lane;  // one row per lane
                    if (m < rows && m < 32 * MSA) {
                        const int64_t row = p0 + m;
                        float x[32];
#pragma unroll
                        for (int i = 0; i < 32; ++i) x[i] = we[m * kEpiStride + i];
                        if constexpr (FP8) {
                            uint32_t cw[8];
                            const int sc = mxfp8_quant_block(x, cw);
                            u32x4 *dst = reinterpret_cast<u32x4 *>(p.o_codes + row * F + fb);
                            dst[0] = (u32x4){cw[0], cw[1], cw[2], cw[3]};
                            dst[1] = (u32x4){cw[4], cw[5], cw[6], cw[7]};
                            p.o_scales[row * (F / 32) + fb / 32] = (uint8_t)sc;
                        } else {
                            uint32_t cw[4];
                            const int sc = mxfp4_quant_block(x, cw);
                            *reinterpret_cast<u32x4 *>(p.o_codes + row * (F / 2) + fb / 2) =
                                (u32x4){cw[0], cw[1], cw[2], cw[3]};
                            p.o_scales[row * (F / 32) + fb / 32] = (uint8_t)sc;
                        }
                        if (p.o_tap) {
                            float4 *t = reinterpret_cast<float4 *>(p.o_tap + row * F + fb);
#pragma unroll
                            for (int i = 0; i < 8; ++i)
                                t[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
                        }
                    }
                }
            }
        } else {
            __syncthreads();  // the y tiles reuse the A tiles' LDS
            float *yt = reinterpret_cast<float *>(lds) + wave * 32 * kYStride;
#pragma unroll
            for (int ms = 0; ms < MSA; ++ms)
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns) {
                    float val[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) val[v] = acc[ms][ns][v];
                    store_y_tile(yt, ms, val, p.out_f32 + nb * kBN + wave * 32 * kNS + 32 * ns);
                }
        }
    };
    if (rows <= 32)
        run(std::integral_constant<int, 1>{});
    else if (rows <= 64)
        run(std::integral_constant<int, 2>{});
    else
        run(std::integral_constant<int, kMS>{});
}

template <bool FP8, bool ROWS, bool GATE_UP>
void launch_t(const GemmArgs &a, bool stream_once, dim3 grid, hipStream_t s) {
    if (stream_once)
        hipLaunchKernelGGL((mx_gemm_kernel<FP8, ROWS, GATE_UP, true>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((mx_gemm_kernel<FP8, ROWS, GATE_UP, false>), grid, dim3(kThreads), 0, s, a);
}

}  // namespace

int32_t mx_gemm_bm() { return kBM; }

bool mx_gemm_supported(int mode, int32_t K, int32_t N, bool gate_up) {
    const int bn = mode != kMxFP4 ? Mx<true>::kBN : Mx<false>::kBN;
    if (K <= 0 || N <= 0 || K % 128) return false;
    if (mode != kMxFP8Rows && K > kMaxK) return false;  // the staged E8M0 row scales
    return gate_up ? (N % 2 == 0 && (N / 2) % (bn / 2) == 0) : N % bn == 0;
}

hipError_t launch_mx_gemm(const GemmArgs &a, int mode, bool gate_up, bool stream_once, int32_t max_tiles,
                          hipStream_t s) {
    const int bn = mode != kMxFP4 ? Mx<true>::kBN : Mx<false>::kBN;
    const int64_t nb = gate_up ? (a.N / 2) / (bn / 2) : a.N / bn;
    const int64_t items = (int64_t)max_tiles * nb;
    const dim3 grid((unsigned)((items + 7) / 8 * 8));
    if (mode == kMxFP8Rows) {
        if (gate_up) launch_t<true, true, true>(a, stream_once, grid, s);
        else launch_t<true, true, false>(a, stream_once, grid, s);
    } else if (mode == kMxFP8) {
        if (gate_up) launch_t<true, false, true>(a, stream_once, grid, s);
        else launch_t<true, false, false>(a, stream_once, grid, s);
    } else {
        if (gate_up) launch_t<false, false, true>(a, stream_once, grid, s);
        else launch_t<false, false, false>(a, stream_once, grid, s);
    }
    return hipGetLastError();
}

}  // namespace moe
