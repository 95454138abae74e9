// permute.hip - stable grouping of the local token-slots by expert, and the M-tile
// list of the grouped GEMMs.
//
// Slot s = t*k + j (token t's j-th routed expert) is local when its expert lies in
// [e_begin, e_end) (one GPU's expert-parallel share; vLLM recipe
// "thinkingmachines/Inkling-2-Small", section "Overview": expert parallelism follows
// the tensor-parallel group). Local slots are ordered by expert and by s within an
// expert (a stable counting sort) in three passes over chunks of consecutive tokens:
//   count   per-chunk histogram (LDS atomics; order does not matter for counts)
//   scan    one workgroup: per-expert running sums over chunks, the exclusive
//           prefix over experts, and the list of BM-row tiles of every expert
//   scatter one wave per chunk walks its slots in order; a ballot over the lanes
//           holding the same expert gives each slot its rank among equal experts,
//           so positions are exact and stable for any routing, duplicates included.
#include "internal.h"

namespace moe {
namespace {

__global__ void __launch_bounds__(256) count_kernel(const int32_t *__restrict__ idx, int32_t n_slots,
                                                    int32_t chunk_slots, int32_t e_begin, int32_t n_loc,
                                                    int32_t *__restrict__ chunk_counts) {
    extern __shared__ int32_t cnt[];
    for (int i = threadIdx.x; i < n_loc; i += 256) cnt[i] = 0;
    __syncthreads();
    const int64_t s0 = (int64_t)blockIdx.x * chunk_slots;
    const int64_t s1 = min<int64_t>(s0 + chunk_slots, n_slots);
    for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) {
        const int el = idx[s] - e_begin;
        if (el >= 0 && el < n_loc) atomicAdd(&cnt[el], 1);
    }
    __syncthreads();
    int32_t *dst = chunk_counts + (int64_t)blockIdx.x * n_loc;
    for (int i = threadIdx.x; i < n_loc; i += 256) dst[i] = cnt[i];
}

constexpr int kScanThreads = 1024;

// In-place exclusive prefix sum of v[0..n) (n <= 4 * kScanThreads) by one workgroup;
// returns the total. part must hold kScanThreads entries.
__device__ int32_t block_exclusive_scan(int32_t *v, int n, int32_t *part) {
    const int tid = threadIdx.x;
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int b = tid * per, e = min(b + per, n);
    int32_t sum = 0;
    for (int i = b; i < e; ++i) sum += v[i];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int32_t add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int32_t run = part[tid] - sum;  // exclusive prefix of this thread's range
    for (int i = b; i < e; ++i) {
        const int32_t x = v[i];
        v[i] = run;
        run += x;
    }
    const int32_t total = part[kScanThreads - 1];
    __syncthreads();
    return total;
}

// In-place exclusive prefix sum of v[0..n) by one workgroup of kSmall threads
// (n <= 4 * kSmall); returns the total. part must hold kScanThreads entries.
template <int kSmall>
__device__ int32_t small_scan_impl(int32_t *v, int n, int32_t *part) {
    const int tid = threadIdx.x;
    const int per = (n + kSmall - 1) / kSmall;
    const int b = tid * per, e = min(b + per, n);
    int32_t sum = 0;
    for (int i = b; i < e; ++i) sum += v[i];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kSmall; off <<= 1) {
        const int32_t add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int32_t run = part[tid] - sum;
    for (int i = b; i < e; ++i) {
        const int32_t x = v[i];
        v[i] = run;
        run += x;
    }
    const int32_t total = part[kSmall - 1];
    __syncthreads();
    return total;
}
__device__ __forceinline__ int32_t small_exclusive_scan(int32_t *v, int n, int32_t *part) {
    return small_scan_impl<256>(v, n, part);
}

__global__ void __launch_bounds__(kScanThreads) scan_kernel(PermuteArgs a) {
    __shared__ int32_t cnt[4096];
    __shared__ int32_t tiles[4096];
    __shared__ int32_t part[kScanThreads];
    const int n = a.n_loc;
    for (int el = threadIdx.x; el < n; el += kScanThreads) {
        int32_t run = 0;
        for (int c = 0; c < a.n_chunks; ++c) {
            int32_t *p = a.chunk_counts + (int64_t)c * n + el;
            const int32_t v = *p;
            *p = run;  // becomes the chunk's base within the expert
            run += v;
        }
        cnt[el] = run;
        a.counts[el] = run;
        tiles[el] = (run + a.bm - 1) / a.bm;
    }
    __syncthreads();
    const int32_t S = block_exclusive_scan(cnt, n, part);
    const int32_t n_tiles = block_exclusive_scan(tiles, n, part);
    for (int el = threadIdx.x; el < n; el += kScanThreads) {
        a.offsets[el] = cnt[el];
        const int32_t t0 = tiles[el];
        const int32_t t1 = el + 1 < n ? tiles[el + 1] : n_tiles;
        for (int32_t t = t0; t < t1; ++t) {
            a.tile_expert[t] = el;
            a.tile_row0[t] = cnt[el] + (t - t0) * a.bm;
        }
    }
    if (threadIdx.x == 0) {
        a.offsets[n] = S;
        a.ctrl->S = S;
        a.ctrl->n_tiles = n_tiles;
    }
}

__global__ void __launch_bounds__(64) scatter_kernel(PermuteArgs a, int32_t n_slots, int32_t chunk_slots) {
    extern __shared__ int32_t cursor[];
    const int lane = threadIdx.x;
    const int n = a.n_loc;
    const int32_t *base = a.chunk_counts + (int64_t)blockIdx.x * n;
    for (int el = lane; el < n; el += 64) cursor[el] = a.offsets[el] + base[el];
    __syncthreads();
    const int64_t s0 = (int64_t)blockIdx.x * chunk_slots;
    const int64_t s1 = min<int64_t>(s0 + chunk_slots, n_slots);
    const uint64_t lt = (1ull << lane) - 1;
    for (int64_t g = s0; g < s1; g += 64) {
        const int64_t s = g + lane;
        const bool valid = s < s1;
        const int el = valid ? a.idx[s] - a.e_begin : -1;
        const bool local = valid && el >= 0 && el < n;
        if (valid && !local) a.slot_pos[s] = -1;
        uint64_t rem = __ballot(local);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int e = __shfl(el, leader);
            const bool mine = local && el == e;
            const uint64_t m = __ballot(mine);
            const int32_t start = __builtin_amdgcn_readfirstlane(cursor[e]);
            if (mine) {
                const int32_t pos = start + __popcll(m & lt);
                a.sorted_slot[pos] = (int32_t)s;
                a.slot_pos[s] = pos;
            }
            if (lane == leader) cursor[e] = start + __popcll(m);
            rem &= ~m;
        }
    }
}

// Whole permutation in one workgroup for small batches (T*k <= 8192 slots, <= 1024
// local experts): per-wave histograms of four contiguous quarters of the slots, the
// exclusive scans and the tile list, then each wave scatters its quarter with the
// ballot ranking, starting from its own per-expert bases. Also clears the control
// block's accumulators, so no separate fill is needed.
constexpr int kSmallThreads = 256;
constexpr int kSmallMaxLocal = 1024;

__global__ void __launch_bounds__(kSmallThreads) permute_small_kernel(PermuteArgs a) {
    __shared__ int32_t cnt[4][kSmallMaxLocal];  // per-wave counts, then per-wave bases
    __shared__ int32_t tot[kSmallMaxLocal];
    __shared__ int32_t tiles[kSmallMaxLocal];
    __shared__ int32_t part[kScanThreads];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n_loc;
    const int32_t n_slots = a.T * a.k;
    const int32_t q = (n_slots + 3) / 4;  // slots per wave quarter
    const int32_t s0 = wave * q, s1 = min(n_slots, s0 + q);
    for (int i = tid; i < 4 * kSmallMaxLocal; i += kSmallThreads) (&cnt[0][0])[i] = 0;
    if (tid == 0) {
        a.ctrl->amax_a = 0;
        a.ctrl->amax_i = 0;
    }
    __syncthreads();
    for (int32_t s = s0 + lane; s < s1; s += 64) {
        const int el = a.idx[s] - a.e_begin;
        if (el >= 0 && el < n) atomicAdd(&cnt[wave][el], 1);
    }
    __syncthreads();
    for (int el = tid; el < n; el += kSmallThreads) {
        int32_t run = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int32_t c = cnt[w][el];
            cnt[w][el] = run;  // base of wave w within the expert
            run += c;
        }
        tot[el] = run;
        a.counts[el] = run;
        tiles[el] = (run + a.bm - 1) / a.bm;
    }
    __syncthreads();
    const int32_t S = small_exclusive_scan(tot, n, part);
    const int32_t n_tiles = small_exclusive_scan(tiles, n, part);
    for (int el = tid; el < n; el += kSmallThreads) {
        a.offsets[el] = tot[el];
        const int32_t t0 = tiles[el];
        const int32_t t1 = el + 1 < n ? tiles[el + 1] : n_tiles;
        for (int32_t t = t0; t < t1; ++t) {
            a.tile_expert[t] = el;
            a.tile_row0[t] = tot[el] + (t - t0) * a.bm;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) cnt[w][el] += tot[el];  // absolute cursors
    }
    if (tid == 0) {
        a.offsets[n] = S;
        a.ctrl->S = S;
        a.ctrl->n_tiles = n_tiles;
    }
    __syncthreads();
    const uint64_t lt = (1ull << lane) - 1;
    int32_t *cursor = cnt[wave];
    for (int32_t gbase = s0; gbase < s1; gbase += 64) {
        const int32_t s = gbase + lane;
        const bool valid = s < s1;
        const int el = valid ? a.idx[s] - a.e_begin : -1;
        const bool local = valid && el >= 0 && el < n;
        if (valid && !local) a.slot_pos[s] = -1;
        uint64_t rem = __ballot(local);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int e = __shfl(el, leader);
            const bool mine = local && el == e;
            const uint64_t m = __ballot(mine);
            const int32_t start = __builtin_amdgcn_readfirstlane(cursor[e]);
            if (mine) {
                const int32_t pos = start + __popcll(m & lt);
                a.sorted_slot[pos] = s;
                a.slot_pos[s] = pos;
            }
            if (lane == leader) cursor[e] = start + __popcll(m);
            rem &= ~m;
        }
    }
}

}  // namespace

bool permute_small_ok(int32_t T, int32_t k, int32_t n_loc) {
    return (int64_t)T * k <= 8192 && n_loc <= kSmallMaxLocal;
}

hipError_t launch_permute_small(const PermuteArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs &a, hipStream_t s) {
    const int32_t n_slots = a.T * a.k;
    const int32_t chunk_slots = a.chunk_tokens * a.k;
    const size_t lds = sizeof(int32_t) * (size_t)a.n_loc;
    hipLaunchKernelGGL(count_kernel, dim3(a.n_chunks), dim3(256), lds, s, a.idx, n_slots, chunk_slots, a.e_begin,
                       a.n_loc, a.chunk_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3(a.n_chunks), dim3(64), lds, s, a, n_slots, chunk_slots);
    return hipGetLastError();
}

}  // namespace moe
