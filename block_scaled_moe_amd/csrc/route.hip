// route.hip - softmax-then-top-k router (vLLM recipe "thinkingmachines/Inkling-2-Small",
// section "Overview": each token is routed to 8 of 384 experts, no shared expert).
//
// Logits: logits[t][e] = sum over d ascending of h[t][d] * wr[e][d] in fp32 from +0.
// Each bf16 product is exact in fp32, so fmaf(h, w, acc) rounds exactly like
// acc + h*w; the fixed order makes the top-k selection a deterministic function of
// the inputs. The kernel is a register-blocked SIMT product: a wave owns TPW tokens
// and 64*EPL experts (lane = expert column), the k loop runs strictly ascending for
// every accumulator, h values are LDS broadcasts and router-weight values are
// conflict-free LDS reads of consecutive experts.
#include "formats.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int KC = 32;

template <int TPW, int EPL>
__global__ void __launch_bounds__(256) router_logits_kernel(int32_t T, int32_t D, int32_t E,
                                                            const uint16_t *__restrict__ h,
                                                            const uint16_t *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ logits,
                                                            uint32_t *__restrict__ amax_bits) {
    constexpr int BT = 4 * TPW;   // tokens per workgroup
    constexpr int BE = 64 * EPL;  // experts per workgroup
    __shared__ float hs[KC][BT];
    __shared__ float ws[KC][BE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
    const bool do_amax = amax_bits != nullptr && blockIdx.y == 0;
    uint32_t amax = 0;

    float acc[TPW][EPL];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < EPL; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < D; k0 += KC) {
        const int kc = min(KC, D - k0);
        // hidden tile: BT tokens x KC values, 4 bf16 per item, stored transposed
        for (int it = tid; it < BT * (KC / 4); it += 256) {
            const int tt = it / (KC / 4), kq = (it % (KC / 4)) * 4;
            const int t = t0 + tt;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (t < T) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kq + i < kc) {
                        const uint16_t b = h[(int64_t)t * D + k0 + kq + i];
                        v[i] = bf16_to_f32(b);
                        amax = max(amax, (uint32_t)(b & 0x7fff));
                    }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) hs[kq + i][tt] = v[i];
        }
        // router-weight tile: BE experts x KC values
        for (int it = tid; it < BE * (KC / 4); it += 256) {
            const int ee = it / (KC / 4), kq = (it % (KC / 4)) * 4;
            const int e = e0 + ee;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (e < E) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kq + i < kc) v[i] = bf16_to_f32(wr[(int64_t)e * D + k0 + kq + i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ws[kq + i][ee] = v[i];
        }
        __syncthreads();
        for (int kk = 0; kk < kc; ++kk) {
            float hv[TPW], wv[EPL];
#pragma unroll
            for (int i = 0; i < TPW; ++i) hv[i] = hs[kk][wave * TPW + i];
#pragma unroll
            for (int j = 0; j < EPL; ++j) wv[j] = ws[kk][lane + 64 * j];
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int j = 0; j < EPL; ++j) acc[i][j] = __builtin_fmaf(hv[i], wv[j], acc[i][j]);
        }
        __syncthreads();
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

// One wave per token: k rounds of a wave-wide arg-max over the not-yet-taken experts,
// then the renormalised softmax weights of the selected logits in fp64.
__global__ void __launch_bounds__(256) router_topk_kernel(int32_t T, int32_t E, int32_t k,
                                                          const float *__restrict__ logits,
                                                          int32_t *__restrict__ idx, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *row = logits + (int64_t)t * E;
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
        int bi = -1;
        for (int e = lane; e < E; e += 64) {
            bool taken = false;
#pragma unroll
            for (int q = 0; q < 8; ++q) taken |= (q < r) && (sel[q] == e);
            if (taken) continue;
            const float v = row[e];
            if (bi < 0 || ranks_before(v, e, bv, bi)) {
                bv = v;
                bi = e;
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
        sel[r] = bi;
        selv[r] = bv;
    }
    if (lane == 0) {
        const double l0 = (double)selv[0];
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += exp((double)selv[j] - l0);
        for (int j = 0; j < k; ++j) {
            idx[(int64_t)t * k + j] = sel[j];
            w[(int64_t)t * k + j] = (float)(exp((double)selv[j] - l0) / den);
        }
    }
}

}  // namespace

hipError_t launch_router_logits(int32_t T, int32_t D, int32_t E, const uint16_t *h, const uint16_t *wr,
                                const float *bias, float *logits, uint32_t *amax_bits, hipStream_t s) {
    if (T >= 8192 && E <= 384) {
        dim3 grid((T + 31) / 32, (E + 383) / 384);
        hipLaunchKernelGGL((router_logits_kernel<8, 6>), grid, dim3(256), 0, s, T, D, E, h, wr, bias, logits,
                           amax_bits);
    } else if (T >= 1024) {
        dim3 grid((T + 15) / 16, (E + 127) / 128);
        hipLaunchKernelGGL((router_logits_kernel<4, 2>), grid, dim3(256), 0, s, T, D, E, h, wr, bias, logits,
                           amax_bits);
    } else {
        dim3 grid((T + 3) / 4, (E + 63) / 64);
        hipLaunchKernelGGL((router_logits_kernel<1, 1>), grid, dim3(256), 0, s, T, D, E, h, wr, bias, logits,
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
