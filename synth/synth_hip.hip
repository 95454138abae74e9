// synth_hip.hip - device twin of the bf16 normal sampler in synth.c.
//
// Input generation only (no part of the MoE layer's arithmetic). It draws the
// same deviates as synth_normal_bf16 in synth.c: SplitMix64 counter outputs,
// sign from bit 63, magnitude by inverse-CDF search over a threshold table that
// the host builds once and passes in. The draw is integer-only, so given the
// same table the bytes are identical to the host's.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9e3779b97f4a7c15ULL;
constexpr int kGuideBits = 16;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

__global__ void __launch_bounds__(256) normal_bf16_kernel(uint64_t key, uint64_t offset, uint64_t count,
                                                          const uint64_t* __restrict__ thr,
                                                          const uint32_t* __restrict__ guide,
                                                          uint16_t* __restrict__ out) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        uint64_t u = mix64(key + (offset + i + 1) * kGamma);
        uint64_t r = u & 0x7fffffffffffffffULL;
        uint32_t c = guide[r >> (63 - kGuideBits)];
        while (r >= thr[c]) ++c;  // thr[n-1] = 2^63 > r ends every search
        out[i] = (uint16_t)(((u >> 63) << 15) | c);
    }
}

}  // namespace

// out[i] = deviate offset+i of the sub-sequence with base state `key`
// (synth_key(seed, stream) on the host). thr/guide/out are device pointers.
extern "C" int synth_hip_normal_bf16(uint64_t key, uint64_t offset, uint64_t count,
                                     const uint64_t* thr, const uint32_t* guide, uint16_t* out,
                                     hipStream_t stream) {
    if (count == 0) return 0;
    if (!thr || !guide || !out) return -1;
    uint64_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(normal_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, key, offset,
                       count, thr, guide, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
