// route.hip - softmax-then-top-k router (vLLM recipe "thinkingmachines/Inkling-2-Small",
// section "Overview": each token is routed to 8 of 384 experts, no shared expert).
//
// Logits: logits[t][e] = sum over d ascending of h[t][d] * wr[e][d] in fp32 from +0.
// Each bf16 product is exact in fp32, so fmaf(h, w, acc) rounds exactly like
// acc + h*w; the fixed order makes the top-k selection a deterministic function of
// the inputs. Each logit is one dependent chain of D FMAs, so the kernel is a
// register-blocked SIMT product: a wave owns TPW tokens and 64*EPL experts (lane =
// expert column), h values are LDS broadcasts, and the K chunks are prefetched two
// ahead into registers and double-buffered in LDS so the chains never wait on memory.
#include "formats.h"
#include "internal.h"

namespace moe {
namespace {

// LDS tiles are row-major with one padding float per row, so a lane per expert reads
// ws[e][k] from distinct banks and the 8-byte stores of 4 consecutive k stay simple.
template <int TPW, int EPL, int KC>
struct RouterCfg {
    static constexpr int BT = 4 * TPW;          // tokens per workgroup
    static constexpr int BE = 64 * EPL;         // experts per workgroup
    static constexpr int HS = KC + 4;           // floats per LDS h row
    static constexpr int WS = KC + 1;           // floats per LDS router-weight row
    static constexpr int H_TOTAL = BT * KC / 4; // 8-byte (4 x bf16) loads per chunk
    static constexpr int W_TOTAL = BE * KC / 4;
    static constexpr int H_ITEMS = (H_TOTAL + 255) / 256;
    static constexpr int W_ITEMS = (W_TOTAL + 255) / 256;
    static constexpr int BUF = BT * HS + BE * WS;  // floats per LDS buffer
};

template <int TPW, int EPL, int KC>
__global__ void __launch_bounds__(256) router_logits_kernel(int32_t T, int32_t D, int32_t E,
                                                            const uint16_t *__restrict__ h,
                                                            const uint16_t *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ logits,
                                                            uint32_t *__restrict__ amax_bits) {
    using C = RouterCfg<TPW, EPL, KC>;
    __shared__ float lds[2][C::BUF];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * C::BT, e0 = blockIdx.y * C::BE;
    const bool do_amax = amax_bits != nullptr && blockIdx.y == 0;
    uint32_t amax = 0;

    float acc[TPW][EPL];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < EPL; ++j) acc[i][j] = 0.0f;

    // two register sets of prefetched 8-byte loads (4 bf16 each); zero past T, E or D
    uint2 rh[2][C::H_ITEMS], rw[2][C::W_ITEMS];
    const int n_chunks = (D + KC - 1) / KC;
    auto load = [&](uint2 (&dh)[C::H_ITEMS], uint2 (&dw)[C::W_ITEMS], int c) {
        const int k0 = c * KC;
#pragma unroll
        for (int i = 0; i < C::H_ITEMS; ++i) {
            const int item = tid + 256 * i;
            const int r = item / (KC / 4), k = k0 + 4 * (item % (KC / 4));
            const int t = t0 + r;
            dh[i] = make_uint2(0, 0);
            if (item < C::H_TOTAL && t < T && k < D) {
                const uint16_t *src = h + (int64_t)t * D + k;
                if (k + 4 <= D && ((reinterpret_cast<uintptr_t>(src) & 7) == 0)) {
                    dh[i] = *reinterpret_cast<const uint2 *>(src);
                } else {
                    uint32_t v[4] = {0, 0, 0, 0};
                    for (int q = 0; q < 4 && k + q < D; ++q) v[q] = src[q];
                    dh[i] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
                }
            }
        }
#pragma unroll
        for (int i = 0; i < C::W_ITEMS; ++i) {
            const int item = tid + 256 * i;
            const int r = item / (KC / 4), k = k0 + 4 * (item % (KC / 4));
            const int e = e0 + r;
            dw[i] = make_uint2(0, 0);
            if (item < C::W_TOTAL && e < E && k < D) {
                const uint16_t *src = wr + (int64_t)e * D + k;
                if (k + 4 <= D && ((reinterpret_cast<uintptr_t>(src) & 7) == 0)) {
                    dw[i] = *reinterpret_cast<const uint2 *>(src);
                } else {
                    uint32_t v[4] = {0, 0, 0, 0};
                    for (int q = 0; q < 4 && k + q < D; ++q) v[q] = src[q];
                    dw[i] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
                }
            }
        }
    };
    auto store = [&](const uint2 (&dh)[C::H_ITEMS], const uint2 (&dw)[C::W_ITEMS], float *buf) {
#pragma unroll
        for (int i = 0; i < C::H_ITEMS; ++i) {
            const int item = tid + 256 * i;
            if (item >= C::H_TOTAL) continue;
            const int r = item / (KC / 4), kq = 4 * (item % (KC / 4));
            float *d = buf + r * C::HS + kq;
            d[0] = __uint_as_float(dh[i].x << 16);
            d[1] = __uint_as_float(dh[i].x & 0xffff0000u);
            d[2] = __uint_as_float(dh[i].y << 16);
            d[3] = __uint_as_float(dh[i].y & 0xffff0000u);
            if (do_amax) {
                amax = max(amax, max(max(dh[i].x & 0x7fffu, (dh[i].x >> 16) & 0x7fffu),
                                     max(dh[i].y & 0x7fffu, (dh[i].y >> 16) & 0x7fffu)));
            }
        }
#pragma unroll
        for (int i = 0; i < C::W_ITEMS; ++i) {
            const int item = tid + 256 * i;
            if (item >= C::W_TOTAL) continue;
            const int r = item / (KC / 4), kq = 4 * (item % (KC / 4));
            float *d = buf + C::BT * C::HS + r * C::WS + kq;
            d[0] = __uint_as_float(dw[i].x << 16);
            d[1] = __uint_as_float(dw[i].x & 0xffff0000u);
            d[2] = __uint_as_float(dw[i].y << 16);
            d[3] = __uint_as_float(dw[i].y & 0xffff0000u);
        }
    };

    load(rh[0], rw[0], 0);
    if (n_chunks > 1) load(rh[1], rw[1], 1);
    for (int c = 0; c < n_chunks; c += 2) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // register set s holds chunk c + s
            const int cc = c + s;
            if (cc >= n_chunks) break;
            float *buf = lds[s];
            store(rh[s], rw[s], buf);
            __syncthreads();
            if (cc + 2 < n_chunks) load(rh[s], rw[s], cc + 2);
            const int kc = min(KC, D - cc * KC);
            const float *hb = buf + (wave * TPW) * C::HS;
            const float *wb = buf + C::BT * C::HS + lane * C::WS;
            // k strictly ascending for every accumulator; full chunks are unrolled so the
            // LDS reads run ahead of the dependent FMA chain
            auto step = [&](int kk) {
                float hv[TPW], wv[EPL];
#pragma unroll
                for (int i = 0; i < TPW; ++i) hv[i] = hb[i * C::HS + kk];
#pragma unroll
                for (int j = 0; j < EPL; ++j) wv[j] = wb[64 * j * C::WS + kk];
#pragma unroll
                for (int i = 0; i < TPW; ++i)
#pragma unroll
                    for (int j = 0; j < EPL; ++j) acc[i][j] = __builtin_fmaf(hv[i], wv[j], acc[i][j]);
            };
            if (kc == KC) {
#pragma unroll 16
                for (int kk = 0; kk < KC; ++kk) step(kk);
            } else {
                for (int kk = 0; kk < kc; ++kk) step(kk);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = t0 + wave * TPW + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = e0 + lane + 64 * j;
            if (e >= E) continue;
            float v = acc[i][j];
            if (bias) v = v + bias[e];
            logits[(int64_t)t * E + e] = v;
        }
    }
    if (do_amax) {
        for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
        if (lane == 0 && amax) atomicMax(amax_bits, amax << 16);
    }
}

// (value, index) a ranks before (value, index) b: larger logit, ties to the lower index
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// One wave per token: the token's logits are read once into registers (expert
// e = lane + 64 i), then k rounds of a wave-wide arg-max over the not-yet-taken experts,
// then the renormalised softmax weights of the selected logits in fp64.
constexpr int kTopkMaxE = 1024;  // experts held in registers (16 per lane)

__global__ void __launch_bounds__(256) router_topk_kernel(int32_t T, int32_t E, int32_t k,
                                                          const float *__restrict__ logits,
                                                          int32_t *__restrict__ idx, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *row = logits + (int64_t)t * E;
    constexpr int PER = kTopkMaxE / 64;
    float v[PER];
    uint32_t live = 0;  // bit i: expert lane + 64 i exists and is not taken
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = 0.f;
        if (e < E) {
            v[i] = row[e];
            live |= 1u << i;
        }
    }
    int sel[8];
    float selv[8];
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
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            if (((live >> i) & 1u) && (bi < 0 || ranks_before(v[i], e, bv, bi))) {
                bv = v[i];
                bi = e;
                bslot = i;
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (oi >= 0 && (bi < 0 || ranks_before(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if (bi >= 0 && (bi & 63) == lane && bslot >= 0) live &= ~(1u << (bi >> 6));
        sel[r] = bi;
        selv[r] = bv;
    }
    // lane j < k computes exp(l_j - l_0); the sum runs in j order on every lane
    double ex = 0.0;
    int my_sel = -1;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (lane == j && j < k) {
            ex = exp((double)selv[j] - (double)selv[0]);
            my_sel = sel[j];
        }
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += __shfl(ex, j);
    if (lane < k) {
        idx[(int64_t)t * k + lane] = my_sel;
        w[(int64_t)t * k + lane] = (float)(ex / den);
    }
}

}  // namespace

hipError_t launch_router_logits(int32_t T, int32_t D, int32_t E, const uint16_t *h, const uint16_t *wr,
                                const float *bias, float *logits, uint32_t *amax_bits, hipStream_t s) {
    if (T >= 8192 && E <= 384) {
        dim3 grid((T + 31) / 32, (E + 383) / 384);
        hipLaunchKernelGGL((router_logits_kernel<8, 6, 16>), grid, dim3(256), 0, s, T, D, E, h, wr, bias, logits,
                           amax_bits);
    } else if (T >= 1024) {
        dim3 grid((T + 15) / 16, (E + 127) / 128);
        hipLaunchKernelGGL((router_logits_kernel<4, 2, 32>), grid, dim3(256), 0, s, T, D, E, h, wr, bias, logits,
                           amax_bits);
    } else {
        dim3 grid((T + 3) / 4, (E + 63) / 64);
        hipLaunchKernelGGL((router_logits_kernel<1, 1, 128>), grid, dim3(256), 0, s, T, D, E, h, wr, bias, logits,
                           amax_bits);
    }
    return hipGetLastError();
}

hipError_t launch_router_topk(int32_t T, int32_t E, int32_t k, const float *logits, int32_t *idx, float *w,
                              hipStream_t s) {
    hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, T, E, k, logits, idx, w);
    return hipGetLastError();
}

}  // namespace moe
