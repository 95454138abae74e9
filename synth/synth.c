/*
 * synth.c - seeded synthetic inputs for the routed-expert MoE layer.
 *
 * This module only draws random numbers. It holds none of the layer's
 * arithmetic (no routing, no quantisation, no GEMM); the CPU oracle and the
 * GPU path consume the bytes it writes.
 *
 * Uniform bits: counter-based SplitMix64 (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014; finaliser
 * constants from Vigna's published splitmix64). The n-th output of
 * sub-sequence (seed, stream) is mix(key(seed, stream) + (n+1)*gamma), so any
 * slice of any tensor can be regenerated alone, in any order, on any device.
 *
 * bf16 normal deviates: value i is drawn from the exact distribution of
 * bf16_RNE(sigma * Z), Z ~ N(0,1), by inverse-CDF sampling over the bf16
 * magnitudes. Bit 63 of the i-th output is the sign; its low 63 bits r are a
 * uniform integer, and the magnitude is the smallest bf16 code c with
 * r < thr[c], where thr[c] = floor(2^63 * P(|sigma Z| < midpoint(c, c+1))).
 * The threshold table is built once in fp64 (erf / erfc); sampling itself is
 * integer-only, so a GPU implementation reproduces these bytes exactly when
 * it is handed the same table. A 2^16-entry guide table (first candidate code
 * per 2^47-wide bucket of r) makes a draw cost one or two comparisons.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9e3779b97f4a7c15ULL
#define SYNTH_GUIDE_BITS 16

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Base state of one (seed, stream) sub-sequence. */
uint64_t synth_key(uint64_t seed, uint64_t stream) {
    return sm_mix(sm_mix(seed + SM_GAMMA) ^ (stream * 0xd1b54a32d192ed03ULL + 0x632be59bd9b4e019ULL));
}

/* The n-th 64-bit output of sub-sequence (seed, stream). */
uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t n) {
    return sm_mix(synth_key(seed, stream) + (n + 1) * SM_GAMMA);
}

static inline double bf16_bits_value(uint32_t c) {
    uint32_t u = c << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Number of magnitude codes in the table for sigma: codes 0..n-1 with v(n-1) >= 10 sigma. */
int32_t synth_table_size(double sigma) {
    uint32_t c = 1;
    while (c < 0x7f80u && bf16_bits_value(c) < 10.0 * sigma) ++c;
    return (int32_t)(c + 1);
}

/* Build thresholds thr[0..n-1] and the 2^16-entry guide table for sigma. */
void synth_build_table(double sigma, int32_t n, uint64_t *thr, uint32_t *guide) {
    const double two63 = 9223372036854775808.0;
    for (int32_t c = 0; c < n - 1; ++c) {
        double mid = 0.5 * (bf16_bits_value((uint32_t)c) + bf16_bits_value((uint32_t)c + 1));
        double y = mid / (sigma * 1.41421356237309504880168872420969808);
        if (y <= 1.0) {
            thr[c] = (uint64_t)floor(erf(y) * two63);
        } else {
            double q = ceil(ldexp(erfc(y), 63));
            thr[c] = (uint64_t)(two63 - q);
        }
    }
    thr[n - 1] = 0x8000000000000000ULL; /* catch-all: every r < 2^63 */
    int32_t c = 0;
    for (uint32_t b = 0; b < (1u << SYNTH_GUIDE_BITS); ++b) {
        uint64_t lo = (uint64_t)b << (63 - SYNTH_GUIDE_BITS);
        while (thr[c] <= lo) ++c;
        guide[b] = (uint32_t)c;
    }
}

static inline uint16_t draw_bf16(uint64_t u, const uint64_t *thr, const uint32_t *guide) {
    uint64_t r = u & 0x7fffffffffffffffULL;
    uint32_t c = guide[r >> (63 - SYNTH_GUIDE_BITS)];
    while (r >= thr[c]) ++c;
    return (uint16_t)(((u >> 63) << 15) | c);
}

/* out[i] = bf16 deviate number offset+i of (seed, stream), i in [0, count). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t count,
                       const uint64_t *thr, const uint32_t *guide, uint16_t *out) {
    const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i) {
        uint64_t u = sm_mix(key + (offset + (uint64_t)i + 1) * SM_GAMMA);
        out[i] = draw_bf16(u, thr, guide);
    }
}

/*
 * Seeded Fisher-Yates permutation of 0..n-1: for i = n-1 down to 1, swap
 * perm[i] with perm[j], j = floor(u * (i+1) / 2^64) for the next 64-bit output u.
 */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t *perm) {
    for (int32_t i = 0; i < n; ++i) perm[i] = i;
    uint64_t c = 0;
    for (int32_t i = n - 1; i > 0; --i) {
        uint64_t u = synth_u64(seed, stream, c++);
        int32_t j = (int32_t)(((unsigned __int128)u * (unsigned __int128)(uint64_t)(i + 1)) >> 64);
        int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
}

/*
 * Zipf-like router bias for the skewed-routing workload: a seeded permutation
 * gives every expert a rank 1..n, and bias[e] = (float)(-slope * ln(rank_e)).
 */
int synth_rank_bias(uint64_t seed, uint64_t stream, int32_t n, double slope, float *bias) {
    int32_t perm[4096];
    if (n < 1 || n > 4096) return -1;
    synth_permutation(seed, stream, n, perm);
    for (int32_t e = 0; e < n; ++e) bias[e] = (float)(-slope * log((double)(perm[e] + 1)));
    return 0;
}
