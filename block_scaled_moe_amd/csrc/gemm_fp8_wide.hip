// gemm_fp8_wide.hip - prefill grouped expert GEMMs for FP8 experts (E4M3 weights with an
// fp32 scale per output channel, activations with a dynamic fp32 scale per row: the fp8
// variant of the vLLM recipe "thinkingmachines/Inkling-Small") on the gfx950 scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4, with 256 x 256 workgroup tiles.
//
// Same operands, lane layout, epilogues and per-element chunk order as the FP8 (ROWS)
// instantiation of mx_gemm_kernel (gemm_mx.hip): every E8M0 scale operand is 127 (2^0),
// the sums are multiplied by fl32(row scale * channel scale) after the K loop, gate_up
// writes the fp32 SwiGLU output; the two give the same bits. The 128-row kernel is bound
// by the operand bytes its loads pull into the CU (weights 16 KiB and activations 8 KiB
// per 64-wide chunk for 32 MFMAs); here each weight operand byte feeds twice the MFMAs:
//  - 8 waves, two per SIMD, as 2 (M) x 4 (N). Wave (wm, wn) computes 4 x 2 MFMA tiles:
//    the 32-row subtiles 2i + wm (i = 0..3) of the tile's 256 rows, interleaved so that a
//    partial tile splits evenly between the two M-waves, and the same 64 weight rows
//    (gate_up: 32 gate rows and the matching up rows) as wave wn of the 128-row kernel;
//  - per 64-wide K chunk the workgroup stages in LDS the chunk's activation codes (80-byte
//    rows: 64 code bytes + 16, conflict-free operand reads) and the codes of its 256 weight
//    rows in the packed layout (a lane's operand is two contiguous 16-byte pieces);
//  - four stages, and every load goes through registers two chunks ahead: chunk c + 2 is
//    loaded while chunk c is multiplied and stored to its stage after chunk c + 1's
//    MFMAs, so each register wait is for loads issued a whole chunk earlier; one barrier
//    per chunk. (Copying the weights straight into LDS with global_load_lds saved the
//    registers, but the compiler then drained every outstanding load before each LDS
//    store, so the ring never filled.)
//  - per chunk the workgroup loads 16 KiB of activations and 16 KiB of weights for 64
//    MFMAs, a third fewer bytes per MFMA than the 128-row tiles.
// Accumulator v of lane l is row 8(v/4) + 4(l/32) + v%4 of its subtile, column l%32.
#include "formats.h"
#include "gemm_common.h"
#include "internal.h"
#include "layout.h"

namespace moe {
namespace {

using namespace gemm_detail;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

#ifndef MOE_FP8W_GROUP
#define MOE_FP8W_GROUP 4  // M-tiles per expert-major work group (gemm_common.h)
#endif
constexpr int kThreads = 512, kBM = 256, kBN = 256, kNS = 2, kGroup = MOE_FP8W_GROUP;
constexpr int kARow = 80;             // LDS bytes per A row: 64 code bytes + 16 (bank spread)
constexpr int kACodes = kBM * kARow;  // A codes [256 rows][80]
constexpr int kBCodes = 8 * 2048;     // B codes [row block 0..7][2 KiB packed block]
constexpr int kStage = kACodes + kBCodes;
static_assert(kStage % 16 == 0 && 4 * kStage <= 160 * 1024, "stage layout");

// Workgroup barrier for the K loop: this wave's LDS accesses complete, then s_barrier.
// __syncthreads() would also wait for every outstanding vector load, draining the ring at
// each chunk; the loads a stage needs are already complete, since their registers are
// waited for before the LDS stores.
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

__device__ __forceinline__ v8i operand(u32x4 lo, u32x4 hi) {
    return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <bool GATE_UP>
__global__ void __launch_bounds__(kThreads, 1) fp8_wide_gemm_kernel(const GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
    __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
    __shared__ __attribute__((aligned(16))) uint8_t st2[kStage];
    __shared__ __attribute__((aligned(16))) uint8_t st3[kStage];

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

    // ---- loads of chunk c into register slot s (past the end of K: the last chunk again,
    // unused): wave w loads row block w's 2 KiB packed block (two 1 KiB instructions);
    // thread t the activation pieces i = t + 512 q (row i / 4, piece i % 4; rows past the
    // tile's end read its first row)
    const uint8_t *wblk = p.w_codes + (int64_t)e * N * K + (int64_t)(rb_row0(wave) >> 5) * kb * 2048 + lane * 16;
    const int piece = t & 3;
    const uint8_t *ap0 = p.a_codes + a_row(t >> 2) * K + 16 * piece;
    const uint8_t *ap1 = p.a_codes + a_row(128 + (t >> 2)) * K + 16 * piece;
    u32x4 a_pf[2][2], b_pf[2][2];
    auto load = [&](int s, int c) __attribute__((always_inline)) {
        c = min(c, n_chunks - 1);
        a_pf[s][0] = *reinterpret_cast<const u32x4 *>(ap0 + 64 * c);
        a_pf[s][1] = *reinterpret_cast<const u32x4 *>(ap1 + 64 * c);
        b_pf[s][0] = *reinterpret_cast<const u32x4 *>(wblk + (int64_t)c * 2048);
        b_pf[s][1] = *reinterpret_cast<const u32x4 *>(wblk + (int64_t)c * 2048 + 1024);
    };
    auto store = [&](uint8_t *stage, int s) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4 *>(stage + (t >> 2) * kARow + 16 * piece) = a_pf[s][0];
        *reinterpret_cast<u32x4 *>(stage + (128 + (t >> 2)) * kARow + 16 * piece) = a_pf[s][1];
        *reinterpret_cast<u32x4 *>(stage + kACodes + wave * 2048 + lane * 16) = b_pf[s][0];
        *reinterpret_cast<u32x4 *>(stage + kACodes + wave * 2048 + 1024 + lane * 16) = b_pf[s][1];
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

        // the MFMAs of the chunk in `stage` (E8M0 scale operands 127: 2^0)
        auto mma = [&](const uint8_t *stage) __attribute__((always_inline)) {
            if constexpr (MSA > 0) {
                v8i bf[kNS];
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns) {
                    const uint8_t *q = stage + kACodes + (ns ? rb1 : rb0) * 2048 + g2 * 512 + l32 * 16;
                    bf[ns] = operand(*reinterpret_cast<const u32x4 *>(q), *reinterpret_cast<const u32x4 *>(q + 1024));
                }
#pragma unroll
                for (int i = 0; i < MSA; ++i) {
                    const uint8_t *ar = stage + (32 * (2 * i + wm) + l32) * kARow + 16 * g2;
                    const v8i af = operand(*reinterpret_cast<const u32x4 *>(ar), *reinterpret_cast<const u32x4 *>(ar + 32));
#pragma unroll
                    for (int ns = 0; ns < kNS; ++ns)
                        acc[i][ns] =
                            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[ns], acc[i][ns], 0, 0, 0, 127, 0, 127);
                }
            }
        };
        // chunk c from `cur`: chunk c + 2 into register slot c % 2 (issued first), the
        // MFMAs, then chunk c + 1 (slot (c + 1) % 2, loaded during chunk c - 1) into `nxt`
        // (its stage last read in chunk c - 3) and the barrier that publishes it
        auto step = [&](const uint8_t *cur, uint8_t *nxt, int c, auto slot_c) __attribute__((always_inline)) {
            constexpr int S = decltype(slot_c)::value;  // c % 2
            load(S, c + 2);
            __builtin_amdgcn_sched_barrier(0);
            if (c < n_chunks) mma(cur);
            __builtin_amdgcn_sched_barrier(0);
            store(nxt, S ^ 1);
            lds_barrier();
        };

        load(0, 0);
        load(1, 1);
        store(st0, 0);
        __syncthreads();
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        // whole ring turns (a branch out of the middle made the compiler spill); the steps
        // of the last turn past the end of K only load (in bounds, unused) and synchronise
        for (int c = 0; c < n_chunks; c += 4) {
            step(st0, st1, c, I0{});
            step(st1, st2, c + 1, I1{});
            step(st2, st3, c + 2, I0{});
            step(st3, st0, c + 3, I1{});
        }

        // ---- epilogue: accumulator v of subtile i = row 32 (2 i + wm) + 8(v/4) + 4 g2 + v%4;
        // the tile's row scales through LDS
        float *rs = reinterpret_cast<float *>(st0);
        __syncthreads();
        if (t < 32 * n_sub) rs[t] = p.a_rscale[a_row(t)];
        __syncthreads();
        if constexpr (MSA > 0) {
            // the outputs leave 32 x 32 at a time through this wave's tile in stage 1, each
            // lane storing 16-byte row pieces (rows past the tile's end are not stored)
            float *yt = reinterpret_cast<float *>(st1) + wave * 32 * kYStride;
            auto put = [&](int i, const float (&val)[16], float *out, int64_t ld, bool nt) __attribute__((always_inline)) {
                __builtin_amdgcn_wave_barrier();  // the previous tile's reads of yt come first
#pragma unroll
                for (int v = 0; v < 16; ++v) yt[(8 * (v / 4) + 4 * g2 + (v % 4)) * kYStride + l32] = val[v];
                __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave complete in issue order
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = (lane >> 3) + 8 * j, q = lane & 7, m = 32 * (2 * i + wm) + r;
                    const float4 x = *reinterpret_cast<const float4 *>(yt + r * kYStride + 4 * q);
                    if (m < rows) store_f4(out + (int64_t)(p0 + m) * ld + 4 * q, x, nt);
                }
            };
            const float *ch = p.w_tscale + (int64_t)e * N;
            if (GATE_UP) {
                const int col0 = nb * (kBN / 2) + wn * 32;
                const float cg = ch[col0 + l32], cu = ch[F + col0 + l32];
#pragma unroll
                for (int i = 0; i < MSA; ++i) {
                    float val[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float sr = rs[32 * (2 * i + wm) + 8 * (v / 4) + 4 * g2 + (v % 4)];
                        val[v] = swiglu(acc[i][0][v] * (sr * cg), acc[i][1][v] * (sr * cu));
                    }
                    put(i, val, p.out_f32 + col0, F, false);
                }
            } else {
#pragma unroll
                for (int ns = 0; ns < kNS; ++ns) {
                    const int n0 = nb * kBN + wn * 64 + 32 * ns;
                    const float cn = ch[n0 + l32];
#pragma unroll
                    for (int i = 0; i < MSA; ++i) {
                        float val[16];
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            val[v] = acc[i][ns][v] * (rs[32 * (2 * i + wm) + 8 * (v / 4) + 4 * g2 + (v % 4)] * cn);
                        put(i, val, p.out_f32 + n0, N, true);  // y: store_y's non-temporal stores
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

int32_t fp8_wide_gemm_bm() { return kBM; }

hipError_t launch_fp8_wide_gemm(const GemmArgs &a, bool gate_up, int32_t max_tiles, hipStream_t s) {
    const int64_t nb = gate_up ? (a.N / 2) / (kBN / 2) : a.N / kBN;
    const int64_t items = (int64_t)max_tiles * nb;
    const dim3 grid((unsigned)((items + 7) / 8 * 8));
    if (gate_up) hipLaunchKernelGGL(fp8_wide_gemm_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(fp8_wide_gemm_kernel<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
