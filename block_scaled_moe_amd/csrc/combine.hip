// combine.hip - weighted combine of the expert outputs (vLLM recipe
// "thinkingmachines/Inkling-2-Small", section "Overview": a token's output is the
// gate-weighted sum over its routed experts; no shared expert).
//
// out[t][n] = sum over j ascending of w[t][j] * y[pos(t, j)][n] for the token's local
// slots, accumulated in fp64 and rounded once to fp32; a token with no local slot gets
// a zero row. A deterministic gather: every output element is written exactly once,
// with no atomics, and each thread moves four consecutive columns (16-byte accesses).
#include "internal.h"

namespace moe {
namespace {

__global__ void __launch_bounds__(256) combine_kernel(int32_t T, int32_t D, int32_t k,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const float *__restrict__ w, const float *__restrict__ y,
                                                      float *__restrict__ out) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one float4 of out
    const int64_t per_row = D / 4;
    if (q >= (int64_t)T * per_row) return;
    const int64_t t = q / per_row;
    const int64_t c = (q % per_row) * 4;
    // all slot positions and weights first (independent loads), then the rows
    int32_t pos[8];
    double wj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pos[j] = j < k ? slot_pos[t * k + j] : -1;
        wj[j] = j < k ? (double)w[t * k + j] : 0.0;
    }
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = pos[j] >= 0 ? *reinterpret_cast<const float4 *>(y + (int64_t)pos[j] * D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (pos[j] < 0) continue;
        a0 += wj[j] * (double)v[j].x;
        a1 += wj[j] * (double)v[j].y;
        a2 += wj[j] * (double)v[j].z;
        a3 += wj[j] * (double)v[j].w;
    }
    *reinterpret_cast<float4 *>(out + t * D + c) = make_float4((float)a0, (float)a1, (float)a2, (float)a3);
}

}  // namespace

hipError_t launch_combine(int32_t T, int32_t D, int32_t k, const int32_t *slot_pos, const float *w, const float *y,
                          float *out, hipStream_t s) {
    const int64_t n = (int64_t)T * (D / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, D, k, slot_pos, w, y,
                       out);
    return hipGetLastError();
}

}  // namespace moe
