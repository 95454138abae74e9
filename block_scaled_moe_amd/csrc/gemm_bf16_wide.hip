// gemm_bf16_wide.hip - prefill grouped expert GEMMs for bf16 experts (the checkpoint's
// unquantised BF16 variant, vLLM recipe "thinkingmachines/Inkling-Small", section
// "Variants") with 256 x 256 workgroup tiles.
//
// Same arithmetic as the bf16 instantiation of tile_gemm_kernel (gemm_tile.hip): the bf16
// weights and activations as stored, v_mfma_f32_32x32x16_bf16 with fp32 accumulation in
// the same chunk and step order, the gate_up output rounded to bf16; the two give the same
// bits. The tile kernel's 64-row M-tiles load each expert's 42 MB gate_up weight panel
// once per tile (three tiles at about 170 rows per expert), and the loop is bound by the
// bytes its loads pull into the CUs; here a weight value is loaded once per 256 rows:
//  - 8 waves, two per SIMD, as 2 (M) x 4 (N). Wave (wm, wn) computes 4 x 2 MFMA tiles:
//    the 32-row subtiles 2i + wm (i = 0..3) of the tile's 256 rows (interleaved, so that
//    a partial tile splits evenly between the two M-waves) and 64 weight rows (gate_up:
//    32 gate rows and the matching up rows);
//  - per 64-wide K chunk the workgroup stages in LDS the activation rows (bf16, 144-byte
//    rows: 128 + 16, conflict-free operand reads) and the bf16 weights of its 256 weight
//    rows as the four 16-byte B operands of the chunk's MFMA steps, [step][g][r], so that
//    each operand read is one contiguous 1 KiB per wave; wave w loads row block w's 4 KiB
//    packed block with four 1 KiB-contiguous instructions and scatters the pieces;
//  - two stages: chunk c + 1 is loaded into registers while chunk c is multiplied, then
//    stored to the other stage; one barrier per chunk.
// Per chunk and workgroup: 32 KiB of weights and 32 KiB of activations loaded for 256
// MFMAs.
// K order inside a chunk as in gemm_tile.hip: lane half g supplies k = 32g + 8s .. + 7 at
// MFMA step s, for both operands. 32x32x16 operand layout: A lane l holds row l%32, B lane
// l column l%32, 8 values each; accumulator v of lane l is row 8(v/4) + 4(l/32) + v%4 of
// its subtile, column l%32.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

using namespace gemm_detail;

typedef float float16_t __attribute__((ext_vector_type(16)));

#ifndef MOE_BFW_GROUP
#define MOE_BFW_GROUP 4  // M-tiles per expert-major work group (gemm_common.h)
#endif
constexpr int kThreads = 512, kBM = 256, kBN = 256, kNS = 2, kGroup = MOE_BFW_GROUP;
constexpr int kARow = 144;            // LDS bytes per activation row: 64 bf16 + 16 (bank spread)
constexpr int kACodes = kBM * kARow;  // activations [256 rows][144]
constexpr int kBBlock = 4096;         // bf16 weights of one 32-row block: [step 4][half 2][row 32][16 B]
constexpr int kStage = kACodes + 8 * kBBlock;
static_assert(kStage % 16 == 0 && 2 * kStage <= 160 * 1024, "stage layout");

// Workgroup barrier for the K loop: this wave's LDS accesses complete, then s_barrier.
// __syncthreads() would also wait for the next chunk's loads, issued before the MFMAs;
// the loads a stage needs are complete, their registers waited for before the stores.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// floats per row of a wave's 32 x 32 output staging tile (16-byte rows; eight waves' tiles
// take 36 KiB of a free stage)
constexpr int kYStride = 36;
__device__ __forceinline__ void store_f4(float *p, float4 v, bool nt) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v x = {v.x, v.y, v.z, v.w};
    if (nt)
        __builtin_nontemporal_store(x, reinterpret_cast<f4v *>(p));
    else
        *reinterpret_cast<f4v *>(p) = x;
}

template <bool GATE_UP>
__global__ void __launch_bounds__(kThreads, 1) bf16_wide_gemm_kernel(const GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
    __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];

    const int K = p.K, N = p.N, F = N / 2;
    const int NB = GATE_UP ? F / (kBN / 2) : N / kBN;

    // ---- work item of this workgroup (XCD-contiguous ranges, as in the tile kernels)
    const int n_tiles = p.ctrl->n_tiles;
    const int per_xcd = (n_tiles * NB + 7) / 8;
    const int b = blockIdx.x;
    if ((b >> 3) >= per_xcd) return;
    int tile, nb;
    if (!expert_major_item<kGroup>((b & 7) * per_xcd + (b >> 3), NB, kBM, n_tiles, p.tile_expert, p.tile_row0,
                                   p.offsets, tile, nb))
        return;

    const int el = p.tile_expert[tile];
    const int p0 = p.tile_row0[tile];
    const int rows = min(kBM, p.offsets[el + 1] - p0);
    const int n_sub = (rows + 31) / 32;  // 32-row subtiles holding rows
    const int e = p.e_begin + el;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, g2 = lane >> 5;
    const int64_t kb = K / 64;
    const int n_chunks = K / 64;
    auto a_row = [&](int r) -> int64_t {
        const int pos = p0 + (r < rows ? r : 0);
        return p.gather_by_token ? p.sorted_slot[pos] / p.top_k : pos;
    };
    // first weight row of the workgroup's row block rb (32 rows)
    auto rb_row0 = [&](int rb) -> int {
        if (GATE_UP) return rb < 4 ? nb * (kBN / 2) + 32 * rb : F + nb * (kBN / 2) + 32 * (rb - 4);
        return nb * kBN + 32 * rb;
    };

    // ---- loads of chunk c (past the end of K: the last chunk again, unused). Wave w: row
    // block w's packed 4 KiB ([half][32 rows][64 B], layout.h), instruction q reading bytes
    // 1024 q + 16 l: half q / 2, row 16 (q % 2) + l / 4, piece l % 4 (MFMA step l % 4);
    // thread t: the 16-byte activation pieces i = t + 512 q (row i / 8, piece i % 8; rows
    // past the tile's end read its first row)
    const int64_t wblk0 = (int64_t)(rb_row0(wave) >> 5) * kb;
    const uint8_t *wc = p.w_codes + (int64_t)e * N * K * 2 + wblk0 * 4096 + lane * 16;
    const uint8_t *a_base = static_cast<const uint8_t *>(p.a_vals);
    const int piece = t & 7;
    int64_t a_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a_off[q] = a_row(64 * q + (t >> 3)) * K * 2 + 16 * piece;
    u32x4 a_pf[4], w_pf[4];
    auto load = [&](int c) __attribute__((always_inline)) {
        c = min(c, n_chunks - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) a_pf[q] = *reinterpret_cast<const u32x4 *>(a_base + a_off[q] + 128 * (int64_t)c);
#pragma unroll
        for (int q = 0; q < 4; ++q) w_pf[q] = *reinterpret_cast<const u32x4 *>(wc + (int64_t)c * 4096 + 1024 * q);
    };
    // the activation pieces as they are; weight piece (half h, row r, step s) to its B
    // operand slot [s][h][r]
    const int w_row = lane >> 2, w_step = lane & 3;
    auto store = [&](uint8_t *stage) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4 *>(stage + (64 * q + (t >> 3)) * kARow + 16 * piece) = a_pf[q];
        uint8_t *bd = stage + kACodes + wave * kBBlock + w_step * 1024;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4 *>(bd + ((q >> 1) * 32 + 16 * (q & 1) + w_row) * 16) = w_pf[q];
    };

    // this wave's weight row blocks (ns = 0, 1)
    const int rb0 = GATE_UP ? wn : 2 * wn, rb1 = GATE_UP ? 4 + wn : 2 * wn + 1;

    auto run = [&](auto msa_c) __attribute__((always_inline)) {
        constexpr int MSA = decltype(msa_c)::value;  // this wave's subtiles holding rows (0..4)
        constexpr int MA = MSA > 0 ? MSA : 1;
        float16_t acc[MA][kNS];
#pragma unroll
        for (int i = 0; i < MA; ++i)
#pragma unroll
            for (int j = 0; j < kNS; ++j) acc[i][j] = (float16_t){};

        // the MFMAs of the chunk in `stage`: four 16-deep steps
        auto mma = [&](const uint8_t *stage) __attribute__((always_inline)) {
            if constexpr (MSA > 0) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 bf[kNS];
#pragma unroll
                    for (int ns = 0; ns < kNS; ++ns)
                        bf[ns] = *reinterpret_cast<const bf16x8 *>(stage + kACodes + (ns ? rb1 : rb0) * kBBlock +
                                                                   s * 1024 + (g2 * 32 + l32) * 16);
#pragma unroll
                    for (int i = 0; i < MSA; ++i) {
                        const bf16x8 af = *reinterpret_cast<const bf16x8 *>(stage + (32 * (2 * i + wm) + l32) * kARow +
                                                                           64 * g2 + 16 * s);
#pragma unroll
                        for (int ns = 0; ns < kNS; ++ns)
                            acc[i][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[ns], acc[i][ns], 0, 0, 0);
                    }
                }
            }
        };
        // chunk c from `cur`: chunk c + 1 into registers (issued first), the MFMAs, then
        // chunk c + 1 into `nxt` (last read in chunk c - 1) and the barrier
        auto step = [&](const uint8_t *cur, uint8_t *nxt, int c) __attribute__((always_inline)) {
            load(c + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (c < n_chunks) mma(cur);
            __builtin_amdgcn_sched_barrier(0);
            store(nxt);
            lds_barrier();
        };

        load(0);
        store(st0);
        __syncthreads();
        // whole pairs of chunks (a branch out of the middle of such a loop made the compiler
        // spill); a step past the end of K only loads (in bounds, unused) and synchronises
        for (int c = 0; c < n_chunks; c += 2) {
            step(st0, st1, c);
            step(st1, st0, c + 1);
        }

        // ---- epilogue: accumulator v of subtile i = row 32 (2 i + wm) + 8(v/4) + 4 g2 + v%4
        if constexpr (MSA > 0) {
            // the outputs leave 32 x 32 at a time through this wave's tile in stage 0 (every
            // wave passed the loop's last barrier), each lane storing 16-byte row pieces (rows
            // past the tile's end are not stored)
            float *yt = reinterpret_cast<float *>(st0) + wave * 32 * kYStride;
            auto stage = [&](const float (&val)[16]) __attribute__((always_inline)) {
                __builtin_amdgcn_wave_barrier();  // the previous tile's reads of yt come first
#pragma unroll
                for (int v = 0; v < 16; ++v) yt[(8 * (v / 4) + 4 * g2 + (v % 4)) * kYStride + l32] = val[v];
                __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave complete in issue order
            };
            if (GATE_UP) {
                // the SwiGLU output rounded to bf16 (nearest even) is the down GEMM's input;
                // lane (r = lane / 4 + 16 j, eighth lane % 4) stores 8 values
                const int f0 = nb * (kBN / 2) + wn * 32;
#pragma unroll
                for (int i = 0; i < MSA; ++i) {
                    float val[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) val[v] = swiglu(acc[i][0][v], acc[i][1][v]);
                    stage(val);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int r = (lane >> 2) + 16 * j, e8 = lane & 3, m = 32 * (2 * i + wm) + r;
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
            } else {
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns) {
                    const int n0 = nb * kBN + wn * 64 + 32 * ns;
#pragma unroll
                    for (int i = 0; i < MSA; ++i) {
                        float val[16];
#pragma unroll
                        for (int v = 0; v < 16; ++v) val[v] = acc[i][ns][v];
                        stage(val);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int r = (lane >> 3) + 8 * j, q = lane & 7, m = 32 * (2 * i + wm) + r;
                            const float4 x = *reinterpret_cast<const float4 *>(yt + r * kYStride + 4 * q);
                            if (m < rows) store_f4(p.out_f32 + (int64_t)(p0 + m) * N + n0 + 4 * q, x, true);
                        }
                    }
                }
            }
        }
    };
    // subtiles 2 i + wm < n_sub; every wave runs the same loads and barriers
    switch ((n_sub - wm + 1) / 2) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
    }
}

}  // namespace

int32_t bf16_wide_gemm_bm() { return kBM; }

bool bf16_wide_gemm_supported(int32_t K, int32_t N, bool gate_up) {
    if (K <= 0 || N <= 0 || K % 64) return false;
    return gate_up ? (N % 2 == 0 && (N / 2) % (kBN / 2) == 0) : N % kBN == 0;
}

hipError_t launch_bf16_wide_gemm(const GemmArgs &a, bool gate_up, int32_t max_tiles, hipStream_t s) {
    const int64_t nb = gate_up ? (a.N / 2) / (kBN / 2) : a.N / kBN;
    const int64_t items = (int64_t)max_tiles * nb;
    const dim3 grid((unsigned)((items + 7) / 8 * 8));
    if (gate_up) hipLaunchKernelGGL(bf16_wide_gemm_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(bf16_wide_gemm_kernel<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
