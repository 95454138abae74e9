// combine.hip - weighted combine of the expert outputs (vLLM recipe
// "thinkingmachines/Inkling-2-Small", section "Overview": a token's output is the
// gate-weighted sum over its routed experts; no shared expert).
//
// out[t][n] = sum over j ascending of w[t][j] * y[pos(t, j)][n] for the token's local
// slots, one fp32 fused multiply-add per slot in slot order; a token with no local
// slot gets a zero row. A deterministic gather: every output element is written
// exactly once, with no atomics.
//
// One workgroup per token: the token's local slot positions and weights are the same for
// the whole workgroup; they are compacted in slot order and one straight-line body per
// count of local slots (0..8) moves 16-byte column groups of the row, all slots' loads of
// two groups issued before the sums.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
typedef float f4v __attribute__((ext_vector_type(4)));

// y is read once and out written once: both marked non-temporal (skewed-mxfp8, whose
// 2.15 GB of y this kernel reads, measured 6.19 -> 6.13 ms per step; no change elsewhere)
__device__ __forceinline__ float4 load_y(const float4 *p) {
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_out(float4 *p, float4 a) {
    __builtin_nontemporal_store((f4v){a.x, a.y, a.z, a.w}, reinterpret_cast<f4v *>(p));
}

// One token's row for its N local slots (positions and weights in slot order): each
// thread moves 16-byte column groups, all N loads of two groups issued before the sums.
template <int N>
__device__ __forceinline__ void combine_row(int n4, const int32_t (&pos)[8], const float (&wj)[8], const float4 *y4,
                                            float4 *o4) {
#pragma unroll 2
    for (int c = threadIdx.x; c < n4; c += kThreads) {
        float4 v[N > 0 ? N : 1];
#pragma unroll
        for (int j = 0; j < N; ++j) v[j] = load_y(y4 + (int64_t)pos[j] * n4 + c);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            acc.x = fmaf(wj[j], v[j].x, acc.x);
            acc.y = fmaf(wj[j], v[j].y, acc.y);
            acc.z = fmaf(wj[j], v[j].z, acc.z);
            acc.w = fmaf(wj[j], v[j].w, acc.w);
        }
        store_out(o4 + c, acc);
    }
}

__global__ void __launch_bounds__(kThreads) combine_kernel(int32_t D, int32_t k,
                                                           const int32_t *__restrict__ slot_pos,
                                                           const float *__restrict__ w,
                                                           const float *__restrict__ y,
                                                           float *__restrict__ out) {
    const int64_t t = blockIdx.x;
    // the token's local slots (position >= 0) compacted in slot order with selects (the
    // values are the same for the whole workgroup)
    int32_t pos[8];
    float wj[8];
    int nl = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        pos[i] = 0;
        wj[i] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int32_t p = j < k ? slot_pos[t * k + j] : -1;
        const float wv = j < k ? w[t * k + j] : 0.0f;
#pragma unroll
        for (int i = 0; i <= j; ++i) {
            const bool here = p >= 0 && nl == i;
            pos[i] = here ? p : pos[i];
            wj[i] = here ? wv : wj[i];
        }
        nl += p >= 0 ? 1 : 0;
    }
    const int n4 = D / 4;
    const float4 *y4 = reinterpret_cast<const float4 *>(y);
    float4 *o4 = reinterpret_cast<float4 *>(out + t * D);
    switch (nl) {
        case 0: combine_row<0>(n4, pos, wj, y4, o4); break;
        case 1: combine_row<1>(n4, pos, wj, y4, o4); break;
        case 2: combine_row<2>(n4, pos, wj, y4, o4); break;
        case 3: combine_row<3>(n4, pos, wj, y4, o4); break;
        case 4: combine_row<4>(n4, pos, wj, y4, o4); break;
        case 5: combine_row<5>(n4, pos, wj, y4, o4); break;
        case 6: combine_row<6>(n4, pos, wj, y4, o4); break;
        case 7: combine_row<7>(n4, pos, wj, y4, o4); break;
        default: combine_row<8>(n4, pos, wj, y4, o4); break;
    }
}

}  // namespace

hipError_t launch_combine(int32_t T, int32_t D, int32_t k, const int32_t *slot_pos, const float *w, const float *y,
                          float *out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(kThreads), 0, s, D, k, slot_pos, w, y, out);
    return hipGetLastError();
}

}  // namespace moe
