// permute.hip - stable grouping of the local token-slots by expert, and the M-tile
// list of the grouped GEMMs.
//
// Slot s = t*k + j (token t's j-th routed expert) is local when its expert lies in
// [e_begin, e_end) (one GPU's expert-parallel share; vLLM recipe
// "thinkingmachines/Inkling-2-Small", section "Overview": expert parallelism follows
// the tensor-parallel group). Local slots are ordered by expert and by s within an
// expert (a stable counting sort) in three passes over chunks of consecutive tokens:
//   count   per-chunk histogram (LDS atomics; order does not matter for counts); extra
//           workgroups of this launch quantise the hidden states (act_quant.h)
//   scan    one workgroup: per-expert running sums over chunks, the exclusive
//           prefix over experts, and the list of BM-row tiles of every expert
//   scatter one wave per chunk walks its slots in groups of 64, in order; within a
//           group each slot's rank among the slots of the same expert comes from
//           comparing the lanes' experts, so positions are exact and stable for any
//           routing, duplicates included.
#include "act_quant.h"
#include "internal.h"

namespace moe {
namespace {

// The hidden-state quantisation carried by a permutation launch: workgroups `first` and
// on quantise blocks in a grid-stride loop (the permutation's own workgroups come first;
// the two jobs share no data, so the launch costs the longer of them instead of both
// plus a launch boundary).
__device__ __forceinline__ void carried_quant(const ActQuant &q, int first) {
    act_quant_range(q, (int64_t)(blockIdx.x - first) * blockDim.x + threadIdx.x, (int64_t)(gridDim.x - first) * blockDim.x);
}

// workgroups of a permutation launch given to the quantisation job
inline int32_t quant_groups(const ActQuant &q, int threads) {
    if (q.fmt == kActNone) return 0;
    const int units = threads / act_quant_unit_threads(q);
    const int64_t g = (act_quant_blocks(q) + units - 1) / units;
    return (int32_t)(g < 1 ? 1 : (g > 2048 ? 2048 : g));
}

// For a group of 64 slots held one per lane (el: local expert, -1 if not local): the
// number of lower lanes holding the same expert (rank) and of all lanes holding it
// (total). One pass per distinct expert of the group: the lanes equal to the lowest
// unhandled lane's expert form a 64-bit mask, which those lanes keep; rank and total
// are bit counts of the kept mask. No LDS traffic inside the loop.
__device__ __forceinline__ void group_rank(int el, int &rank, int &total) {
    uint64_t rem = __ballot(el >= 0);
    uint32_t mlo = 0, mhi = 0;
    while (rem) {
        const int leader = __ffsll((unsigned long long)rem) - 1;
        const int e = __builtin_amdgcn_readlane(el, leader);
        const bool mine = el == e;
        const uint64_t m = __ballot(mine);
        mlo = mine ? (uint32_t)m : mlo;
        mhi = mine ? (uint32_t)(m >> 32) : mhi;
        rem &= ~m;
    }
    rank = (int)__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
    total = __popc(mlo) + __popc(mhi);
}

// Stable placement of one group of 64 consecutive slots (slot s on lane s - group
// start; valid: s in range). cursor[e] is the next free position of local expert e for
// this wave and is advanced by the group's count; each lane reads it before the
// group's first lane of that expert writes it back (LDS accesses of one wave complete
// in order).
__device__ __forceinline__ void place_group(const PermuteArgs &a, int32_t *cursor, int64_t s, bool valid) {
    const int el0 = valid ? a.idx[s] - a.e_begin : -1;
    const bool local = valid && el0 >= 0 && el0 < a.n_loc;
    const int el = local ? el0 : -1;
    int rank, total;
    group_rank(el, rank, total);
    if (valid && !local) a.slot_pos[s] = -1;
    const int32_t start = local ? cursor[el] : 0;
    if (local) {
        const int32_t pos = start + rank;
        a.sorted_slot[pos] = (int32_t)s;
        a.slot_pos[s] = pos;
    }
    __builtin_amdgcn_wave_barrier();
    if (local && rank == 0) cursor[el] = start + total;
}

__global__ void __launch_bounds__(256) count_kernel(const int32_t *__restrict__ idx, int32_t n_slots,
                                                    int32_t chunk_slots, int32_t e_begin, int32_t n_loc,
                                                    int32_t *__restrict__ chunk_counts, Ctrl *__restrict__ ctrl,
                                                    int32_t n_chunks, const ActQuant quant) {
    if ((int32_t)blockIdx.x >= n_chunks) {  // the carried hidden-state quantisation
        carried_quant(quant, n_chunks);
        return;
    }
    extern __shared__ int32_t cnt[];
    for (int i = threadIdx.x; i < n_loc; i += 256) cnt[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {  // accumulators of the later passes
        ctrl->amax_a = 0;
        ctrl->amax_i = 0;
    }
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
constexpr int kSmallWaves = 8;  // waves of the one-workgroup permutation
constexpr int kSmallThreads = 64 * kSmallWaves;

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
    return small_scan_impl<kSmallThreads>(v, n, part);
}

__global__ void __launch_bounds__(kScanThreads) scan_kernel(PermuteArgs a) {
    __shared__ int32_t cnt[4096];
    __shared__ int32_t tiles[4096];
    __shared__ int32_t part[kScanThreads];
    const int n = a.n_loc;
    // Each expert's column of chunk counts is split into `segs` runs of `len` chunks,
    // one thread per (expert, run), so the column walk is spread over the workgroup.
    const int segs = n < kScanThreads ? kScanThreads / n : 1;
    const int len = (a.n_chunks + segs - 1) / segs;
    int32_t *run_sum = tiles;  // [segs][n] run totals, then run bases (n * segs <= 4096)
    for (int u = threadIdx.x; u < n * segs; u += kScanThreads) {
        const int el = u % n, c0 = (u / n) * len, c1 = min(c0 + len, a.n_chunks);
        const int32_t *p = a.chunk_counts + el;
        int32_t sum = 0;
#pragma unroll 16
        for (int c = c0; c < c1; ++c) sum += p[(int64_t)c * n];
        run_sum[u] = sum;
    }
    __syncthreads();
    for (int el = threadIdx.x; el < n; el += kScanThreads) {
        int32_t run = 0;
        for (int r = 0; r < segs; ++r) {
            const int32_t v = run_sum[r * n + el];
            run_sum[r * n + el] = run;
            run += v;
        }
        cnt[el] = run;
    }
    __syncthreads();
    // each chunk count becomes the chunk's base within its expert; loads of a batch
    // are issued before its stores
    for (int u = threadIdx.x; u < n * segs; u += kScanThreads) {
        const int el = u % n, c0 = (u / n) * len, c1 = min(c0 + len, a.n_chunks);
        int32_t *p = a.chunk_counts + el;
        int32_t run = run_sum[u];
        for (int c = c0; c < c1; c += 16) {
            int32_t v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = c + j < c1 ? p[(int64_t)(c + j) * n] : 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (c + j < c1) p[(int64_t)(c + j) * n] = run;
                run += v[j];
            }
        }
    }
    __syncthreads();
    for (int el = threadIdx.x; el < n; el += kScanThreads) {
        a.counts[el] = cnt[el];
        tiles[el] = (cnt[el] + a.bm - 1) / a.bm;
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
    for (int64_t g = s0; g < s1; g += 64) place_group(a, cursor, g + lane, g + lane < s1);
}

// Whole permutation in one workgroup for small batches (T*k <= 8192 slots, <= 1024
// local experts): per-wave histograms of kSmallWaves contiguous parts of the slots, the
// exclusive scans and the tile list, then each wave places its part group by group,
// starting from its own per-expert bases. Also clears the control block's
// accumulators, so no separate fill is needed. Workgroups 1 and on quantise the hidden
// states (act_quant.h).
constexpr int kSmallMaxLocal = 1024;

__global__ void __launch_bounds__(kSmallThreads) permute_small_kernel(PermuteArgs a) {
    if (blockIdx.x > 0) {  // the carried hidden-state quantisation
        carried_quant(a.quant, 1);
        return;
    }
    __shared__ int32_t cnt[kSmallWaves][kSmallMaxLocal];  // per-wave counts, then per-wave bases
    __shared__ int32_t tot[kSmallMaxLocal];
    __shared__ int32_t tiles[kSmallMaxLocal];
    __shared__ int32_t part[kScanThreads];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n_loc;
    const int32_t n_slots = a.T * a.k;
    const int32_t q = (n_slots + kSmallWaves - 1) / kSmallWaves;  // slots per wave
    const int32_t s0 = wave * q, s1 = min(n_slots, s0 + q);
    for (int i = tid; i < kSmallWaves * kSmallMaxLocal; i += kSmallThreads) (&cnt[0][0])[i] = 0;
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
        for (int w = 0; w < kSmallWaves; ++w) {
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
        for (int w = 0; w < kSmallWaves; ++w) cnt[w][el] += tot[el];  // absolute cursors
    }
    if (tid == 0) {
        a.offsets[n] = S;
        a.ctrl->S = S;
        a.ctrl->n_tiles = n_tiles;
    }
    __syncthreads();
    int32_t *cursor = cnt[wave];
    for (int32_t g = s0; g < s1; g += 64) place_group(a, cursor, g + lane, g + lane < s1);
}

}  // namespace

bool permute_small_ok(int32_t T, int32_t k, int32_t n_loc) {
    return (int64_t)T * k <= 8192 && n_loc <= kSmallMaxLocal;
}

hipError_t launch_permute_small(const PermuteArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1 + quant_groups(a.quant, kSmallThreads)), dim3(kSmallThreads), 0, s,
                       a);
    return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs &a, hipStream_t s) {
    const int32_t n_slots = a.T * a.k;
    const int32_t chunk_slots = a.chunk_tokens * a.k;
    const size_t lds = sizeof(int32_t) * (size_t)a.n_loc;
    hipLaunchKernelGGL(count_kernel, dim3(a.n_chunks + quant_groups(a.quant, 256)), dim3(256), lds, s, a.idx, n_slots,
                       chunk_slots, a.e_begin, a.n_loc, a.chunk_counts, a.ctrl, a.n_chunks, a.quant);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3(a.n_chunks), dim3(64), lds, s, a, n_slots, chunk_slots);
    return hipGetLastError();
}

}  // namespace moe
