// route.hip - softmax-then-top-k router (vLLM recipe "thinkingmachines/Inkling-2-Small",
// section "Overview": each token is routed to 8 of 384 experts, no shared expert).
//
// The specified logit is logits[t][e] = sum over d ascending of h[t][d] * wr[e][d] in
// fp32 from +0 (each bf16 product is exact in fp32, so fmaf(h, w, acc) rounds exactly
// like acc + h*w), plus bias[e]. Top-k is by (logit desc, index asc) and the weights
// are the fp64 softmax of the selected logits renormalised over the k. Each logit is a
// dependent chain of D FMAs, so computing all T*E of them is VALU-bound; two paths:
//
//  exact (small T, or when the caller asks for all logits): one expert per lane and one
//    token per workgroup, h broadcast from an fp32 copy in LDS, the router weight read
//    from an expert-fastest bf16 copy (coalesced 16-byte loads, L2-resident); the top k
//    is selected in the same kernel from the row of logits in LDS.
//
//  screened (large T): all logits approximated by a bf16 MFMA GEMM (exact products,
//    fp32 sums in the hardware's order), then per token a rigorous bound on the gap to
//    the sequential sum keeps only experts that can still reach the top k; their logits
//    are recomputed by the exact chain and the top k chosen among them. The bound: both
//    sums approximate S = sum_d p_d with |fl(S) - S| <= gamma_D sum_d |p_d| for any
//    summation order (unit 2^-24 for the sequential RNE chain, 2^-23 allowed for the
//    MFMA's internal rounding), plus D * 2^-124 for denormal flushes, and
//    sum_d |p_d| <= ||h_t|| ||w_e|| (Cauchy-Schwarz). If lo_e <= logit_e <= hi_e and
//    theta is the k-th largest lo, at least k experts have logit >= theta, so the k-th
//    largest logit is >= theta and every expert with hi_e < theta lies strictly below
//    it; the top k (ties included) are therefore among {e : hi_e >= theta}, and the
//    selection there is the same as over all experts. Indices and weights are
//    bit-identical to the exact path.
#include "formats.h"
#include "internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxE = 1024;       // experts supported by the selection kernels
constexpr int kScreenMinT = 512;  // tokens from which the screened path is used
constexpr int kScreenMaxE = 512;  // experts up to which it is (LDS of the selection)

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// (value, index) a ranks before (value, index) b: larger logit, ties to the lower index
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// ---- router weight copy with the expert index fastest: wk8 bf16 [D/8][Ep][8], zero
// past E (3 MiB at 384 x 4096: it stays in every XCD's L2); wpart fp64 [D/64][Ep]
// partial sums of w^2 (optional); also zeroes the max |h| accumulator for the kernels
// that follow. One thread per (expert, 64-wide K block): it reads one full line of its
// row, and consecutive threads write consecutive experts.
__global__ void __launch_bounds__(256) router_prep_kernel(int32_t D, int32_t E, int32_t Ep,
                                                          const uint16_t *__restrict__ wr, uint16_t *__restrict__ wk8,
                                                          double *__restrict__ wpart, uint32_t *__restrict__ amax_bits) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (amax_bits && e == 0 && blockIdx.y == 0) *amax_bits = 0u;  // max |h| accumulates from here
    if (e >= Ep) return;
    const int k0 = 64 * blockIdx.y;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = e < E ? *reinterpret_cast<const u32x4 *>(wr + (int64_t)e * D + k0 + 8 * i) : (u32x4){0u, 0u, 0u, 0u};
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<u32x4 *>(wk8 + ((int64_t)(k0 / 8 + i) * Ep + e) * 8) = v[i];
        const uint32_t q4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double lo = bf_lo(q4[q]), hi = bf_hi(q4[q]);
            ss += lo * lo + hi * hi;
        }
    }
    if (wpart) wpart[(int64_t)blockIdx.y * Ep + e] = ss;
}

#ifndef MOE_CHAIN_RING
#define MOE_CHAIN_RING 4  // weight blocks (32 k each) in the exact chain's register ring
#endif
static_assert(MOE_CHAIN_RING % 2 == 0, "h buffers alternate with the ring slots");
constexpr int kChainKB = 32;  // k per block of the exact chain
// blocks of padding past the end of the expert-fastest weight copy and of the chain's LDS
// h row: the chain runs whole ring turns (up to R - 1 blocks past the last) and loads R - 1
// blocks ahead of the block it computes
constexpr int kChainPadBlocks = 2 * MOE_CHAIN_RING;

// ---- exact logits: a workgroup = one wave = one token x 64 experts, one chain per lane,
// k ascending (grid T x Ep/64, so a decode batch spreads its Ep/64 chains per token over
// the whole chip instead of one CU per token). The token's h row is staged in LDS as
// fp32 (all lanes read the same address, a broadcast); the weights stream from the
// L2-resident bf16 copy through a four-block register ring (blocks of 32 k, loaded three
// blocks ahead). A wave issues about one instruction per four cycles whatever its kind,
// so the loop keeps to the FMA, the widening of each weight and few others: each lane's
// weight pointer advances by a constant stride per block, and the ring's loads ahead of
// the last block read padding blocks of the weight copy and of the LDS row (values never
// used) instead of clamping their block index. Logits go to lg_ws [T][Ep] (for the
// selection kernel) and/or to the caller's logits [T][E]; the workgroups of expert group
// 0 also fold max |h|.
__global__ void __launch_bounds__(64) router_chain_kernel(int32_t D, int32_t E, int32_t Ep,
                                                          const uint16_t *__restrict__ h,
                                                          const uint16_t *__restrict__ wk8,
                                                          const float *__restrict__ bias, float *__restrict__ lg_ws,
                                                          float *__restrict__ logits,
                                                          uint32_t *__restrict__ amax_bits) {
    extern __shared__ __attribute__((aligned(16))) float hrow[];  // [D + padding blocks]
    const int lane = threadIdx.x;
    const int t = blockIdx.x, e = blockIdx.y * 64 + lane;  // e < Ep
    const uint16_t *hp = h + (int64_t)t * D;
    uint32_t amax = 0;
    for (int kk = 8 * lane; kk < D; kk += 8 * 64) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(hp + kk);
        *reinterpret_cast<float4 *>(hrow + kk) = make_float4(bf_lo(x.x), bf_hi(x.x), bf_lo(x.y), bf_hi(x.y));
        *reinterpret_cast<float4 *>(hrow + kk + 4) = make_float4(bf_lo(x.z), bf_hi(x.z), bf_lo(x.w), bf_hi(x.w));
        amax = max(amax, max(max(x.x & 0x7fffu, (x.x >> 16) & 0x7fffu), max(x.y & 0x7fffu, (x.y >> 16) & 0x7fffu)));
        amax = max(amax, max(max(x.z & 0x7fffu, (x.z >> 16) & 0x7fffu), max(x.w & 0x7fffu, (x.w >> 16) & 0x7fffu)));
    }
    if (amax_bits && blockIdx.y == 0) {
        for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
        if (lane == 0 && amax) atomic_max_grow(amax_bits, amax << 16);
    }
    __syncthreads();
    constexpr int KB = kChainKB, R = MOE_CHAIN_RING, NQ = KB / 8;
    const int nb = D / KB;  // D % 64 == 0: even
    // this lane's expert in k-octet 0 (u32x4 units: one k-octet holds Ep pieces); octet q of
    // a block is q * Ep further, and the pointer advances one block per load
    const u32x4 *wsrc = reinterpret_cast<const u32x4 *>(wk8) + e;
    const int64_t oct = Ep, blk = (int64_t)NQ * Ep;
    float acc = 0.0f;
    u32x4 wq[R][NQ];       // weight ring, R blocks
    float4 hq[2][KB / 4];  // h of the current and the next block (read from LDS one block ahead)
    auto load = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) wq[slot][q] = wsrc[q * oct];
        wsrc += blk;
    };
    auto hload = [&](int buf, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < KB / 4; ++q) hq[buf][q] = *reinterpret_cast<const float4 *>(hrow + b * KB + 4 * q);
    };
    auto compute = [&](int slot, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float4 x0 = hq[buf][2 * q], x1 = hq[buf][2 * q + 1];
            const u32x4 y = wq[slot][q];
            acc = __builtin_fmaf(x0.x, bf_lo(y.x), acc);
            acc = __builtin_fmaf(x0.y, bf_hi(y.x), acc);
            acc = __builtin_fmaf(x0.z, bf_lo(y.y), acc);
            acc = __builtin_fmaf(x0.w, bf_hi(y.y), acc);
            acc = __builtin_fmaf(x1.x, bf_lo(y.z), acc);
            acc = __builtin_fmaf(x1.y, bf_hi(y.z), acc);
            acc = __builtin_fmaf(x1.z, bf_lo(y.w), acc);
            acc = __builtin_fmaf(x1.w, bf_hi(y.w), acc);
        }
    };
    // block b sits in weight slot b % R and h buffer b % 2. Whole ring turns, each step's
    // prefetches pinned in place (a conditional use would let the compiler sink them into
    // it); only the compute of blocks past the last, on the final turn, is skipped.
#pragma unroll
    for (int r = 0; r < R - 1; ++r) load(r);
    hload(0, 0);
    for (int b0 = 0; b0 < nb; b0 += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            __builtin_amdgcn_sched_barrier(0);
            load((r + R - 1) % R);  // block b0 + r + R - 1 (past the end: padding)
            hload((r + 1) & 1, b0 + r + 1);
            __builtin_amdgcn_sched_barrier(0);  // the next block's h reads go out first
            if (b0 + r < nb) compute(r, r & 1);
        }
    }
    const float lg = e < E ? (bias ? acc + bias[e] : acc) : 0.0f;
    if (lg_ws) lg_ws[(int64_t)t * Ep + e] = lg;
    if (logits && e < E) logits[(int64_t)t * E + e] = lg;
}

// ---- top-k of exact logit rows: one wave per token, k rounds of a wave-wide arg-max
// (larger logit first, ties to the lower index), then the fp64 softmax weights over the
// k selected: lane j < k computes exp(l_j - l_0) and the sum runs in j order.
template <int PER>  // logits per lane: Ep / 64
__global__ void __launch_bounds__(256) router_topk_kernel(int32_t T, int32_t E, int32_t Ep, int32_t k,
                                                          const float *__restrict__ lg_ws, int32_t *__restrict__ idx,
                                                          float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float v[PER];
    uint32_t live = 0;  // bit i: expert lane + 64 i exists and is not taken
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int ee = lane + 64 * i;
        v[i] = 0.f;
        if (ee < E) {
            v[i] = lg_ws[(int64_t)t * Ep + ee];
            live |= 1u << i;
        }
    }
    float selv[8];
    int sel[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        sel[r] = -1;
        selv[r] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (r >= k) break;
        float bv = 0.f;
        int bi = -1, bslot = -1;
        // selects only (no divergent branches): take a candidate that exists and ranks
        // before the current best (an empty best, index -1, ranks after everything)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ee = lane + 64 * i;
            const bool take = (((live >> i) & 1u) != 0) & ((bi < 0) | (v[i] > bv) | ((v[i] == bv) & (ee < bi)));
            bv = take ? v[i] : bv;
            bi = take ? ee : bi;
            bslot = take ? i : bslot;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            const bool take = (oi >= 0) & ((bi < 0) | (ov > bv) | ((ov == bv) & (oi < bi)));
            bv = take ? ov : bv;
            bi = take ? oi : bi;
        }
        const bool mine = (bi >= 0) & ((bi & 63) == lane) & (bslot >= 0);
        live = mine ? (live & ~(1u << (bi >> 6))) : live;
        sel[r] = bi;
        selv[r] = bv;
    }
    // lane j < k takes the j-th selection (selects, so the k exps run in parallel)
    float my_v = selv[0];
    int my_sel = sel[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        my_v = lane == j ? selv[j] : my_v;
        my_sel = lane == j ? sel[j] : my_sel;
    }
    const double ex = lane < k ? exp((double)my_v - (double)selv[0]) : 0.0;
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += __shfl(ex, j);
    if (lane < k) {
        idx[(int64_t)t * k + lane] = my_sel;
        w[(int64_t)t * k + lane] = (float)(ex / den);
    }
}

// ---- approximate logits by bf16 MFMA: workgroup = 32 kRM tokens x 128 experts, wave =
// 32 kRM x 32 (kRM v_mfma_f32_32x32x16_bf16 tiles sharing each weight fragment, so a
// weight fragment loaded from L2 serves kRM token tiles); K in 64-wide chunks with the same k
// permutation for both operands (lane half g supplies k = 32g + 8s for step s). The h
// tile goes through a double-buffered LDS tile; the weight fragments are 16-byte
// coalesced loads from wk8. Workgroups of the first expert tile also write
// hn[t] = sum h^2 (fp64) and max |h|; those of the first token tile write
// wn[e] = ||w_e|| rounded up, from the partial sums.
constexpr int kHStride = 64 * 2 + 16;  // LDS bytes per h row
#ifndef MOE_ROUTER_RM
#define MOE_ROUTER_RM 2
#endif
constexpr int kRM = MOE_ROUTER_RM;  // 32-token MFMA subtiles per workgroup (and per wave)

__global__ void __launch_bounds__(256) router_mfma_kernel(int32_t T, int32_t D, int32_t Ep, int32_t n_parts,
                                                          const uint16_t *__restrict__ h,
                                                          const uint16_t *__restrict__ wk8,
                                                          const double *__restrict__ wpart, float *__restrict__ lt,
                                                          double *__restrict__ hn, float *__restrict__ wn,
                                                          uint32_t *__restrict__ amax_bits) {
    __shared__ __attribute__((aligned(16))) uint8_t hs[2][32 * kRM * kHStride];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g2 = lane >> 5;
    const int t0 = blockIdx.x * 32 * kRM;
    const int e = blockIdx.y * 128 + wave * 32 + l32;  // this lane's expert (B column)
    const bool stats = blockIdx.y == 0;

    if (blockIdx.x == 0 && tid < 128) {
        const int ee = blockIdx.y * 128 + tid;
        double ss = 0.0;
        for (int p = 0; p < n_parts; ++p) ss += wpart[(int64_t)p * Ep + ee];
        // sqrt and the fp32 rounding each lose < 1 ulp; the factor keeps it an upper bound
        wn[ee] = (float)(sqrt(ss) * (1.0 + 0x1p-20));
    }

    // h staging: thread (row r + 32 i, 16-byte piece q) of the 32 kRM x 64 chunk
    const int r = tid >> 3, q = tid & 7;
    const uint16_t *hsrc[kRM];
    bool hlive[kRM];
#pragma unroll
    for (int i = 0; i < kRM; ++i) {
        hsrc[i] = h + (int64_t)min(t0 + r + 32 * i, T - 1) * D + 8 * q;
        hlive[i] = t0 + r + 32 * i < T;
    }
    const int hdst = r * kHStride + 16 * q;
    const uint16_t *bsrc = wk8 + (int64_t)e * 8 + (int64_t)(4 * g2) * Ep * 8;  // k = 32 g2 within the chunk
    const int64_t bstep = (int64_t)Ep * 8;  // one k-octet

    double ss[kRM] = {};
    uint32_t amax = 0;
    float16_t acc[kRM] = {};
    const int n_chunks = D / 64;
    // software pipeline: chunk c + kRing is loaded (h pieces and weight fragments into
    // ring slot c % kRing) while chunk c is multiplied, so about kRing - 1 chunks of
    // loads are in flight; the h pieces of chunk c + 1 go to the other LDS buffer at
    // the end of chunk c. Loads past the end repeat the last chunk (in bounds, unused).
#ifndef MOE_ROUTER_RING
#define MOE_ROUTER_RING 2
#endif
    constexpr int kRing = MOE_ROUTER_RING;
    u32x4 hreg[kRing][kRM];
    u32x4 breg[kRing][4];
    auto load = [&](int slot, int c) {
#pragma unroll
        for (int i = 0; i < kRM; ++i) hreg[slot][i] = *reinterpret_cast<const u32x4 *>(hsrc[i] + 64 * c);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            breg[slot][s] = *reinterpret_cast<const u32x4 *>(bsrc + (int64_t)(8 * c + s) * bstep);
    };
    auto stage = [&](int buf, int slot) {
#pragma unroll
        for (int i = 0; i < kRM; ++i)
            *reinterpret_cast<u32x4 *>(hs[buf] + hdst + 32 * i * kHStride) = hreg[slot][i];
    };
#pragma unroll
    for (int r = 0; r < kRing; ++r) load(r, min(r, n_chunks - 1));
    stage(0, 0);
    __syncthreads();
    for (int c0 = 0; c0 < n_chunks; c0 += kRing) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            const int c = c0 + j;
            if (c >= n_chunks) break;
            if (stats) {
#pragma unroll
                for (int i = 0; i < kRM; ++i) {
                    if (!hlive[i]) continue;
                    const uint32_t w4[4] = {hreg[j][i].x, hreg[j][i].y, hreg[j][i].z, hreg[j][i].w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float a = bf_lo(w4[u]), b = bf_hi(w4[u]);
                        ss[i] += (double)a * a + (double)b * b;
                        amax = max(amax, max(w4[u] & 0x7fffu, (w4[u] >> 16) & 0x7fffu));
                    }
                }
            }
            const uint8_t *abuf = hs[c & 1];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 bf = __builtin_bit_cast(bf16x8, breg[j][s]);
#pragma unroll
                for (int i = 0; i < kRM; ++i) {
                    const bf16x8 af =
                        *reinterpret_cast<const bf16x8 *>(abuf + (32 * i + l32) * kHStride + 64 * g2 + 16 * s);
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[i], 0, 0, 0);
                }
            }
            // LDS buffer (c + 1) % 2 was last read in chunk c - 1, before the previous barrier
            stage((c + 1) & 1, (j + 1) % kRing);
            load(j, min(c + kRing, n_chunks - 1));
            __syncthreads();
        }
    }
    // accumulator v of lane l: token row 32 i + 8(v/4) + 4 g2 + v%4, expert column l32
#pragma unroll
    for (int i = 0; i < kRM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = t0 + 32 * i + 8 * (v / 4) + 4 * g2 + (v % 4);
            if (t < T) lt[(int64_t)t * Ep + e] = acc[i][v];
        }
    if (stats) {
        // the 8 threads of a row hold its partial sums (lanes 8r'..8r'+7 of the wave)
#pragma unroll
        for (int i = 0; i < kRM; ++i) {
            for (int off = 1; off < 8; off <<= 1) ss[i] += __shfl_xor(ss[i], off);
            if (q == 0 && hlive[i]) hn[t0 + r + 32 * i] = ss[i];
        }
        for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
        if (lane == 0 && amax && amax_bits) atomic_max_grow(amax_bits, amax << 16);
    }
}

// ---- screened selection: 16 lanes per token, 4 tokens per wave, 16 per workgroup.
//  1. bounds lo/hi of every logit from the MFMA value (see the header), theta = k-th
//     largest lo; candidates {e : hi_e >= theta} compacted into LDS;
//  2. exact sequential chains: each wave spreads the (token, candidate) pairs of its 4
//     tokens over its 64 lanes, one chain per lane and pass; the union of the
//     workgroup's candidate experts is staged chunk by chunk (32 k) from the row-major
//     router weight into LDS with contiguous loads, so the chains read weights and h
//     from LDS; each exact logit goes to the token's row of `lt` (no longer needed);
//  3. per token, the 16 lanes keep sorted best-k lists of its exact logits, then k
//     rounds of a 16-lane arg-max over the lists' heads, then the fp64 weights.
// Dynamic LDS: candidate lists [16][E] int16, union slot map [E] int16, expert of each
// slot [E] int16, two weight stages [E][kSelRow] (bf16) and two h stages [16][kSelRowH]
// (fp32: the h values are widened once when staged instead of by each of the token's 16
// lanes at every step; measured 2% off the 8K-token prefill step).
#ifndef MOE_SEL_K
#define MOE_SEL_K 32
#endif
constexpr int kSelK = MOE_SEL_K;       // k per staged chunk
constexpr int kSelP = kSelK / 8;       // 16-byte pieces per staged row
constexpr int kSelRow = 2 * kSelK + 16;  // LDS bytes per staged row: the padding spreads the
                                         // 16-byte pieces of rows at random slots over banks
#ifndef MOE_SEL_TOK
#define MOE_SEL_TOK 16
#endif
constexpr int kSelTok = MOE_SEL_TOK;        // tokens per workgroup (16 lanes each)
constexpr int kSelRowH = 4 * kSelK + 16;   // LDS bytes per staged (fp32) h row
constexpr int kSelThreads = 16 * kSelTok;   // threads per workgroup
// union rows staged at a time: about 150 candidate experts for 16 tokens at decode-like
// spreads; a larger union is processed in windows of kSelCap rows. Sizing the stages by
// the cap instead of E frees LDS for a third workgroup per CU.
#ifndef MOE_SEL_CAP
#define MOE_SEL_CAP 224
#endif
constexpr int kSelCap = MOE_SEL_CAP;
constexpr int kSelItems = (kSelCap * kSelP + kSelTok * kSelP + kSelThreads - 1) / kSelThreads;  // staged pieces per thread

size_t select_lds_bytes(int32_t E) {
    const size_t e2 = (size_t)(E + 1) / 2 * 2;  // keeps the byte arrays 4-byte aligned
    const size_t cap = E < kSelCap ? (size_t)E : (size_t)kSelCap;
    return kSelTok * e2 * 2 + 2 * e2 * 2 + 16 + 2 * cap * kSelRow + 2 * kSelTok * kSelRowH;
}

#ifndef MOE_SEL_OCC
#define MOE_SEL_OCC 3  // waves per SIMD for up to 384 experts (LDS: three workgroups per CU)
#endif
template <int PER>
constexpr int sel_occupancy() { return PER <= 24 ? MOE_SEL_OCC : 2; }

template <int PER>  // logits per lane: ceil(E / 16)
__global__ void __launch_bounds__(kSelThreads, (sel_occupancy<PER>())) router_select_kernel(int32_t T, int32_t D, int32_t E, int32_t Ep, int32_t k,
                                                            const uint16_t *__restrict__ h,
                                                            const uint16_t *__restrict__ wr, float *__restrict__ lt,
                                                            const double *__restrict__ hn,
                                                            const float *__restrict__ wn,
                                                            const float *__restrict__ bias, int32_t *__restrict__ idx,
                                                            float *__restrict__ w) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int e2 = (E + 1) / 2 * 2;
    int16_t *cand = reinterpret_cast<int16_t *>(lds);  // [kSelTok][e2]
    int16_t *uslot = cand + kSelTok * e2;              // [e2]: staged slot of expert e
    int16_t *urow = uslot + e2;                        // [e2]: expert of staged slot s
    // byte offsets from the LDS base (pointer arithmetic on the __shared__ array keeps
    // the accesses ds_* instead of flat)
    const int cap = min(E, kSelCap);                   // union rows per staged window
    uint8_t *wst = lds + ((size_t)((kSelTok + 2) * e2 * 2) + 15) / 16 * 16;  // [2][cap][kSelRow]
    uint8_t *hst = wst + 2 * (size_t)cap * kSelRow;    // [2][kSelTok][kSelRowH]
    __shared__ int32_t n_union, pass_max;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, j = lane & 15;
    const int tl = wave * 4 + grp;
    const int t = blockIdx.x * kSelTok + tl;
    const bool live = t < T;
    const int tt = live ? t : T - 1;
    for (int i = tid; i < e2; i += kSelThreads) uslot[i] = -1;
    if (tid == 0) pass_max = 0;

    // ---- 1. bounds and candidates
    const double u = 0x1p-24;
    const double gam = (double)D * u / (1.0 - (double)D * u) + (double)D * 2 * u / (1.0 - (double)D * 2 * u);
    const double hnorm = sqrt(hn[tt]) * (1.0 + 0x1p-30);
    float *lrow = lt + (int64_t)tt * Ep;
    auto bound = [&](float Lf, float bf, float wnf, float &lo, float &hi) {
        const double L = Lf;
        const double b = bf;
        const double d = gam * hnorm * (double)wnf + (double)D * 0x1p-124;
        const double rad = d + 0x1p-23 * (fabs(L) + fabs(b) + d) + 0x1p-149;
        const double mlo = L + b - rad, mhi = L + b + rad;
        lo = (float)(mlo - fabs(mlo) * 0x1p-23 - 0x1p-149);  // rounds to a value <= mlo
        hi = (float)(mhi + fabs(mhi) * 0x1p-23 + 0x1p-149);  // rounds to a value >= mhi
    };
    float lo[PER], hi[PER];
    uint64_t taken = 0;
    {
        // all loads first (clamped indices, no branches), so they are in flight together
        float Lv[PER], Bv[PER], Wv[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ec = min(j + 16 * i, E - 1);
            Lv[i] = lrow[ec];
            Bv[i] = bias ? bias[ec] : 0.0f;
            Wv[i] = wn[ec];
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            lo[i] = hi[i] = -INFINITY;
            if (j + 16 * i < E) bound(Lv[i], Bv[i], Wv[i], lo[i], hi[i]);
            else taken |= 1ull << i;
        }
    }
    float theta = -INFINITY;
    for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (!((taken >> i) & 1ull) && (bi < 0 || lo[i] > bv)) {
                bv = lo[i];
                bi = i;
            }
        int bl = bi < 0 ? -1 : j;
        for (int off = 8; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 16);
            const int ol = __shfl_xor(bl, off, 16);
            if (ol >= 0 && (bl < 0 || ov > bv || (ov == bv && ol < bl))) {
                bv = ov;
                bl = ol;
            }
        }
        if (bl == j && bi >= 0) taken |= 1ull << bi;
        theta = bv;
    }
    __syncthreads();  // uslot cleared, pass_max zeroed
    int n = 0;  // candidates of this lane's token (uniform in the 16-lane group)
    int16_t *my_cand = cand + tl * e2;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = j + 16 * i;
        const bool flag = live && e < E && hi[i] >= theta;
        const uint32_t bits = (uint32_t)(__ballot(flag) >> (16 * grp)) & 0xffffu;
        if (flag) {
            my_cand[n + __popc(bits & ((1u << j) - 1u))] = (int16_t)e;
            uslot[e] = 0;  // member of the union (slots assigned below)
        }
        n += __popc(bits);
    }
    // pairs of the wave: group g's candidates are pairs [off_g, off_g + n_g)
    int ng[4], og[4], pw = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        ng[g] = __shfl(n, 16 * g);
        og[g] = pw;
        pw += ng[g];
    }
    if (lane == 0) atomicMax(&pass_max, (pw + 63) / 64);
    __syncthreads();
    // slots of the union in expert order (wave 0: running count over 64-expert groups)
    if (tid < 64) {
        int base = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + tid;
            const bool in = e < E && uslot[e] == 0;
            const uint64_t m = __ballot(in);
            if (in) {
                const int sl = base + __popcll(m & ((1ull << tid) - 1ull));
                uslot[e] = (int16_t)sl;
                urow[sl] = (int16_t)e;
            }
            base += __popcll(m);
        }
        if (tid == 0) n_union = base;
    }
    __syncthreads();
    const int nu = n_union, n_pass = pass_max;

    // ---- 2. exact chains over LDS-staged rows, the union in windows of at most cap rows
    const int n_chunks = D / kSelK;
    // chunk c + kSelRing - 1 is loaded into register slot (c - 1) % kSelRing while chunk
    // c is multiplied, so two chunks of loads are in flight; a slot goes to the other LDS
    // buffer one chunk before its use. Loads past the end repeat the last chunk.
#ifndef MOE_SEL_RING
#define MOE_SEL_RING 2
#endif
    constexpr int kSelRing = MOE_SEL_RING;
    const int n_win = (nu + cap - 1) / cap;
    for (int win = 0; win < n_win; ++win) {
        const int r0 = win * cap, nw = min(cap, nu - r0);  // union slots [r0, r0 + nw)
        const int items = (nw + kSelTok) * kSelP;  // 16-byte pieces per chunk: weight rows, then h rows
        u32x4 sreg[kSelRing][kSelItems];
        int32_t src_row[kSelItems];  // the staged row of each item: an expert, else a token
#pragma unroll
        for (int i = 0; i < kSelItems; ++i) {
            const int it = tid + kSelThreads * i, row = it / kSelP;
            src_row[i] = it >= items ? 0 : row < nw ? urow[r0 + row] : min(blockIdx.x * kSelTok + (row - nw), T - 1);
        }
        auto load_chunk = [&](int slot, int c) {
#pragma unroll
            for (int i = 0; i < kSelItems; ++i) {
                const int it = tid + kSelThreads * i;
                const int row = it / kSelP, q = it % kSelP;
                if (it < items) {
                    const uint16_t *src = (row < nw ? wr : h) + (int64_t)src_row[i] * D;
                    sreg[slot][i] = *reinterpret_cast<const u32x4 *>(src + c * kSelK + 8 * q);
                }
            }
        };
        auto store_chunk = [&](int buf, int slot) {
#pragma unroll
            for (int i = 0; i < kSelItems; ++i) {
                const int it = tid + kSelThreads * i;
                const int row = it / kSelP, q = it % kSelP;
                if (it < items) {
                    if (row >= nw) {  // h piece: 8 values widened to fp32
                        const u32x4 v = sreg[slot][i];
                        float4 *dst = reinterpret_cast<float4 *>(hst + (buf * kSelTok + (row - nw)) * kSelRowH + 32 * q);
                        dst[0] = make_float4(bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y));
                        dst[1] = make_float4(bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w));
                    } else {
                        *reinterpret_cast<u32x4 *>(wst + ((size_t)buf * cap + row) * kSelRow + 16 * q) = sreg[slot][i];
                    }
                }
            }
        };
        for (int pass = 0; pass < n_pass; ++pass) {
            const int pr = lane + 64 * pass;  // this lane's pair
            const bool mine = pr < pw;
            int g = 0;
#pragma unroll
            for (int q = 1; q < 4; ++q)
                if (pr >= og[q]) g = q;
            const int ptl = wave * 4 + g;                             // the pair's token in the workgroup
            const int pe = mine ? cand[ptl * e2 + (pr - og[g])] : 0;  // and expert
            const int ps = mine ? uslot[pe] : 0;
            const bool in_win = mine && ps >= r0 && ps < r0 + nw;     // its row is staged in this window
            const int wsl = in_win ? ps - r0 : 0;
            float a = 0.0f;
#pragma unroll
            for (int r = 0; r < kSelRing; ++r) load_chunk(r, min(r, n_chunks - 1));
            store_chunk(0, 0);
            __syncthreads();
            for (int c0 = 0; c0 < n_chunks; c0 += kSelRing) {
#pragma unroll
                for (int jj = 0; jj < kSelRing; ++jj) {
                    const int c = c0 + jj;  // register slot jj held chunk c; LDS buffer c % 2 holds it
                    if (c >= n_chunks) break;
                    const int buf = c & 1;
                    const uint8_t *hrow = hst + (buf * kSelTok + ptl) * kSelRowH;
                    const uint8_t *wrow = wst + ((size_t)buf * cap + wsl) * kSelRow;
#pragma unroll
                    for (int q = 0; q < kSelP; ++q) {
                        const u32x4 wv = *reinterpret_cast<const u32x4 *>(wrow + 16 * q);
                        const float4 h0 = *reinterpret_cast<const float4 *>(hrow + 32 * q);
                        const float4 h1 = *reinterpret_cast<const float4 *>(hrow + 32 * q + 16);
                        a = __builtin_fmaf(h0.x, bf_lo(wv.x), a);
                        a = __builtin_fmaf(h0.y, bf_hi(wv.x), a);
                        a = __builtin_fmaf(h0.z, bf_lo(wv.y), a);
                        a = __builtin_fmaf(h0.w, bf_hi(wv.y), a);
                        a = __builtin_fmaf(h1.x, bf_lo(wv.z), a);
                        a = __builtin_fmaf(h1.y, bf_hi(wv.z), a);
                        a = __builtin_fmaf(h1.z, bf_lo(wv.w), a);
                        a = __builtin_fmaf(h1.w, bf_hi(wv.w), a);
                    }
                    // buffer buf ^ 1 was last read in chunk c - 1, before the previous barrier
                    store_chunk(buf ^ 1, (jj + 1) % kSelRing);
                    load_chunk(jj, min(c + kSelRing, n_chunks - 1));
                    __syncthreads();
                }
            }
            // exact logit of the pair into its token's lt row, at the candidate's position
            const int pt = blockIdx.x * kSelTok + ptl;
            if (in_win && pt < T) lt[(int64_t)pt * Ep + (pr - og[g])] = bias ? a + bias[pe] : a;
        }
    }
    // the barrier waits for the stores of the exact logits (write-through, so they are in
    // this XCD's L2); phase 1 read the same rows through this CU's L1, which the barrier
    // does not invalidate, so L1 is invalidated here and the values read with agent-scope
    // loads
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // ---- 3. per token: sorted best-k lists of the 16 lanes, then merged
    float bestv[8];
    int besti[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        bestv[s] = -INFINITY;
        besti[s] = -1;
    }
    for (int c = j; c < n; c += 16) {
        float v = __hip_atomic_load(lrow + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int vi = my_cand[c];
        // insert into the sorted list: pos = entries that rank before it; the tail moves
        // down one slot (the last falls off) and pos takes the new entry. Written with
        // selects only (a conditional-swap chain here was compiled wrongly on gfx950: the
        // new head was lost when a lane's loop ran a second time).
        int pos = 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) pos += (besti[s] >= 0 && ranks_before(bestv[s], besti[s], v, vi)) ? 1 : 0;
        if (pos < k) {
#pragma unroll
            for (int s = 7; s >= 1; --s) {
                const bool down = s > pos;
                bestv[s] = down ? bestv[s - 1] : bestv[s];
                besti[s] = down ? besti[s - 1] : besti[s];
            }
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                bestv[s] = s == pos ? v : bestv[s];
                besti[s] = s == pos ? vi : besti[s];
            }
        }
    }
    float selv[8];
    int sel[8];
    for (int r = 0; r < 8; ++r) {
        selv[r] = 0.0f;
        sel[r] = -1;
    }
    for (int r = 0; r < k; ++r) {
        float bv = bestv[0];
        int bi = besti[0];
        for (int off = 8; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 16);
            const int oi = __shfl_xor(bi, off, 16);
            if (oi >= 0 && (bi < 0 || ranks_before(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if (bi >= 0 && besti[0] == bi) {  // pop the winner's head
#pragma unroll
            for (int s = 0; s < 7; ++s) {
                bestv[s] = bestv[s + 1];
                besti[s] = besti[s + 1];
            }
            bestv[7] = -INFINITY;
            besti[7] = -1;
        }
        selv[r] = bv;
        sel[r] = bi;
    }
    // lane j < k computes exp(l_j - l_0); the sum runs in j order on every lane
    double ex = 0.0;
    int my_sel = -1;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        if (j == r && r < k) {
            ex = exp((double)selv[r] - (double)selv[0]);
            my_sel = sel[r];
        }
    double den = 0.0;
    for (int r = 0; r < k; ++r) den += __shfl(ex, r, 16);
    if (live && j < k) {
        idx[(int64_t)t * k + j] = my_sel;
        w[(int64_t)t * k + j] = (float)(ex / den);
    }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

RoutePlan route_plan(int32_t T, int32_t D, int32_t E) {
    RoutePlan p{};
    p.screen = T >= kScreenMinT && E <= kScreenMaxE;
    p.Ep = p.screen ? (E + 127) / 128 * 128 : (E + 63) / 64 * 64;
    p.n_parts = D / 64;
    size_t off = 0;
    auto take = [&](size_t n) {
        const size_t o = off;
        off += align256(n);
        return o;
    };
    p.off_wk8 = take((size_t)(D + kChainPadBlocks * kChainKB) * p.Ep * 2);  // + the chain's padding blocks
    if (!p.screen) p.off_exact = take((size_t)T * p.Ep * 4);  // exact logits for the selection
    if (p.screen) {
        p.off_logits = take((size_t)T * p.Ep * 4);  // the MFMA approximations
        p.off_wpart = take((size_t)p.n_parts * p.Ep * 8);
        p.off_hn = take((size_t)T * 8);
        p.off_wn = take((size_t)p.Ep * 4);
    }
    p.bytes = off;
    return p;
}

hipError_t launch_route(const RoutePlan &p, int32_t T, int32_t D, int32_t E, int32_t k, const uint16_t *h,
                        const uint16_t *wr, const float *bias, float *logits_out, int32_t *idx, float *w,
                        uint32_t *amax_bits, void *workspace, hipStream_t s) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint16_t *wk8 = reinterpret_cast<uint16_t *>(ws + p.off_wk8);
    float *scratch = p.screen ? reinterpret_cast<float *>(ws + p.off_logits) : nullptr;
    double *wpart = p.screen ? reinterpret_cast<double *>(ws + p.off_wpart) : nullptr;
    hipLaunchKernelGGL(router_prep_kernel, dim3((unsigned)((p.Ep + 255) / 256), (unsigned)(D / 64)), dim3(256), 0, s,
                       D, E, p.Ep, wr, wk8, wpart, amax_bits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // exact logits (to `out` if given) and, with idx, the top k of each row
    auto exact = [&](float *out, int32_t *ix, float *wt, uint32_t *amax) {
        float *lg_ws = ix ? reinterpret_cast<float *>(ws + p.off_exact) : nullptr;
        hipLaunchKernelGGL(router_chain_kernel, dim3((unsigned)T, (unsigned)(p.Ep / 64)), dim3(64),
                           (size_t)(D + kChainPadBlocks * kChainKB) * 4, s, D, E, p.Ep, h, wk8, bias, lg_ws, out,
                           amax);
        hipError_t e2 = hipGetLastError();
        if (e2 != hipSuccess || !ix) return e2;
        const dim3 grid((unsigned)((T + 3) / 4)), block(256);
        if (p.Ep <= 128)
            hipLaunchKernelGGL((router_topk_kernel<2>), grid, block, 0, s, T, E, p.Ep, k, lg_ws, ix, wt);
        else if (p.Ep <= 384)
            hipLaunchKernelGGL((router_topk_kernel<6>), grid, block, 0, s, T, E, p.Ep, k, lg_ws, ix, wt);
        else
            hipLaunchKernelGGL((router_topk_kernel<kMaxE / 64>), grid, block, 0, s, T, E, p.Ep, k, lg_ws, ix, wt);
        return hipGetLastError();
    };
    if (!p.screen) return exact(logits_out, idx, w, amax_bits);
    double *hn = reinterpret_cast<double *>(ws + p.off_hn);
    float *wn = reinterpret_cast<float *>(ws + p.off_wn);
    hipLaunchKernelGGL(router_mfma_kernel, dim3((unsigned)((T + 32 * kRM - 1) / (32 * kRM)), (unsigned)(p.Ep / 128)),
                       dim3(256), 0, s,
                       T, D, p.Ep, p.n_parts, h, wk8, wpart, scratch, hn, wn, amax_bits);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    {
        const dim3 grid((unsigned)((T + kSelTok - 1) / kSelTok));
        const size_t lds = select_lds_bytes(E);
        if (E <= 128)
            hipLaunchKernelGGL((router_select_kernel<8>), grid, dim3(kSelThreads), lds, s, T, D, E, p.Ep, k, h, wr, scratch,
                               hn, wn, bias, idx, w);
        else if (E <= 256)
            hipLaunchKernelGGL((router_select_kernel<16>), grid, dim3(kSelThreads), lds, s, T, D, E, p.Ep, k, h, wr, scratch,
                               hn, wn, bias, idx, w);
        else if (E <= 384)
            hipLaunchKernelGGL((router_select_kernel<24>), grid, dim3(kSelThreads), lds, s, T, D, E, p.Ep, k, h, wr, scratch,
                               hn, wn, bias, idx, w);
        else
            hipLaunchKernelGGL((router_select_kernel<32>), grid, dim3(kSelThreads), lds, s, T, D, E, p.Ep, k, h, wr, scratch,
                               hn, wn, bias, idx, w);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (logits_out) return exact(logits_out, nullptr, nullptr, nullptr);  // all exact logits on request
    return hipSuccess;
}

}  // namespace moe
