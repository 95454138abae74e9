/*
 * oracle.c - plain, slow CPU oracle of the routed-expert MoE layer with
 * block-scaled (NVFP4 / MXFP8 / MXFP4) experts.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg call into this file. It shares no code, header, table or
 * constant generator with the HIP library, and the HIP library never calls it.
 *
 * Sources (web pages, cited by title and section):
 *  [R] vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview":
 *      384 routed experts, top-8, no shared expert; NVFP4 experts in layers
 *      0-39 and MXFP8 experts in layers 40-47; EP follows the TP group.
 *  [A] AI Primer, "Thinking Machines releases Inkling 2 Small weights under
 *      Apache 2.0": section "TL;DR" (the NVFP4 quantiser maps each block's
 *      maximum to 4 and to 6 and keeps the lower-error result) and section
 *      "NVFP4 and MXFP8 experts" (eight of 384 experts per token; activations
 *      quantised to match the layer's weight format).
 *  [V] vLLM recipe "thinkingmachines/Inkling-Small", section "Variants" and the
 *      recipe's variant list: an OCP MXFP4 checkpoint for AMD Instinct, run on
 *      MI355X as native W4A4 MXFP4 MoE (the MXFP4 format below); and on Hopper the
 *      NVFP4 checkpoint run as W4A16, its weights dequantised to bf16 on the fly
 *      (format 4 below: activations stay bf16, the SwiGLU output is rounded to bf16).
 * The pages fix neither the gate, the expert MLP, the element/scale formats'
 * bit layouts nor the arithmetic order. The readings taken here (softmax then
 * top-8 with lower-index tie-break; SwiGLU experts; E2M1 codes with an E4M3
 * scale per 16 and an fp32 tensor scale amax/(6*448); E4M3 codes with an E8M0
 * scale 2^(floor(log2 amax) - 8) per 32; for MXFP4, E2M1 codes with an E8M0
 * scale 2^(floor(log2 amax) - 2) per 32, activations quantised the same way (the
 * OCP MX shared-exponent rule with E2M1's largest exponent 2, as MXFP8 uses E4M3's 8);
 * fp32 logits summed in ascending k;
 * fp64 expert arithmetic) are the plainest ones the rest supports.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off (no -ffast-math, no FTZ),
 * so every float expression below is one IEEE-754 binary32 operation with
 * round-to-nearest-even, and every double one is binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* ------------------------------------------------------------------------- */
/* Element and scale formats (OCP 8-bit and MX conventions).                  */
/* ------------------------------------------------------------------------- */

/* E2M1: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0; no inf/NaN. */
double orc_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3 "FN": sign bit 7, exponent bits 6-3 (bias 7), mantissa bits 2-0; no
 * infinities; S.1111.111 is NaN; largest finite 448, subnormals m * 2^-9. */
double orc_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0: an unsigned power-of-two exponent, bias 127; 0xFF is NaN. */
double orc_e8m0_value(int code) {
    if ((code & 0xff) == 0xff) return NAN;
    return ldexp(1.0, (code & 0xff) - 127);
}

/*
 * Round |v| to the nearest of the ascending non-negative values tab[0..n-1]
 * (codes 0..n-1), ties to the even code, saturating at tab[n-1]. Plain
 * search; the code's low bit is the mantissa's low bit in both formats, so
 * "even code" is round-half-to-even.
 */
static int nearest_code(double a, const double *tab, int n) {
    if (!(a < tab[n - 1])) return n - 1; /* also catches a == max */
    int lo = 0, hi = n - 1;              /* tab[lo] <= a < tab[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (tab[mid] <= a) lo = mid; else hi = mid;
    }
    double dlo = a - tab[lo], dhi = tab[hi] - a; /* exact: all values are short */
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1) ? hi : lo;
}

static double g_e2m1_pos[8];
static double g_e4m3_pos[127]; /* codes 0x00..0x7E: every finite non-negative value */
static int g_tables_ready = 0;

static void init_tables(void) {
    if (g_tables_ready) return;
    for (int c = 0; c < 8; ++c) g_e2m1_pos[c] = orc_e2m1_value(c);
    for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = orc_e4m3_value(c);
    g_tables_ready = 1;
}

/* E2M1 round-to-nearest-even, saturating to +-6; the sign of v is kept (-0 -> 0x8). */
int orc_e2m1_encode(double v) {
    init_tables();
    int c = nearest_code(fabs(v), g_e2m1_pos, 8);
    return signbit(v) ? (c | 8) : c;
}

/* E4M3 round-to-nearest-even, saturating to +-448 (never NaN); sign kept. */
int orc_e4m3_encode(double v) {
    init_tables();
    int c = nearest_code(fabs(v), g_e4m3_pos, 127);
    return signbit(v) ? (c | 0x80) : c;
}

/* floor(log2(a)) of a positive finite a, from frexp (a = f * 2^x, f in [0.5, 1)). */
static int floor_log2(double a) {
    int x;
    frexp(a, &x);
    return x - 1;
}

/* MXFP8 block scale code for a block maximum: E8M0 of 2^(floor(log2 amax) - 8),
 * the exponent clamped to [-127, 127]; amax == 0 gives code 0x00. */
int orc_e8m0_code_for_amax(float amax) {
    if (!(amax > 0.0f)) return 0;
    int se = floor_log2((double)amax) - 8;
    if (se < -127) se = -127;
    if (se > 127) se = 127;
    return se + 127;
}

/* MXFP4 block scale code: E8M0 of 2^(floor(log2 amax) - 2), the exponent clamped
 * to [-127, 127]; amax == 0 gives code 0x00. */
int orc_mxfp4_scale_code(float amax) {
    if (!(amax > 0.0f)) return 0;
    int se = floor_log2((double)amax) - 2;
    if (se < -127) se = -127;
    if (se > 127) se = 127;
    return se + 127;
}

/* ------------------------------------------------------------------------- */
/* NVFP4 quantiser with the 4-vs-6 block rule ([A] "TL;DR").                  */
/* ------------------------------------------------------------------------- */

/* One candidate: map the block maximum r (already divided by the tensor
 * scale) to M; returns the fp32 squared error and fills codes and scale. */
static float nvfp4_candidate(const float *x, float r, float sg, float M, uint8_t *q, uint8_t *scode) {
    float t = r / M;
    int sc = orc_e4m3_encode((double)t);
    float sdec = (float)orc_e4m3_value(sc); /* exact: E4M3 values are binary32 values */
    float S = sdec * sg;
    float err = 0.0f;
    for (int i = 0; i < 16; ++i) {
        int c;
        if (sdec == 0.0f) {
            c = signbit(x[i]) ? 8 : 0;
        } else {
            float y = x[i] / S;
            c = orc_e2m1_encode((double)y);
        }
        float deq = (float)orc_e2m1_value(c) * S;
        float e = x[i] - deq;
        err = err + e * e;
        q[i] = (uint8_t)c;
    }
    *scode = (uint8_t)sc;
    return err;
}

/*
 * Quantise one block of 16 values given the tensor scale sg. Writes 8 code
 * bytes (element 2i in the low nibble of byte i) and one E4M3 scale byte;
 * returns 1 if the "max -> 4" candidate was kept, 0 for "max -> 6".
 * mode 0: the 4-vs-6 rule; mode 1: always max -> 6 (plain NVFP4);
 * mode 2: always max -> 4.
 */
static int nvfp4_block(const float *x, float sg, int mode, uint8_t *codes8, uint8_t *scale) {
    float amax = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float r = amax / sg;
    uint8_t q6[16], q4[16], s6, s4;
    float err6 = nvfp4_candidate(x, r, sg, 6.0f, q6, &s6);
    float err4 = nvfp4_candidate(x, r, sg, 4.0f, q4, &s4);
    int take4 = err4 < err6; /* equal errors keep the standard max -> 6 mapping */
    if (mode == 1) take4 = 0;
    if (mode == 2) take4 = 1;
    const uint8_t *q = take4 ? q4 : q6;
    for (int i = 0; i < 8; ++i) codes8[i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
    *scale = take4 ? s4 : s6;
    return take4;
}

/* Tensor scale: fp32 amax / (6 * 448), or 1 for an all-zero tensor. */
float orc_nvfp4_tensor_scale(float amax) {
    return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

/*
 * NVFP4-quantise a [rows, K] fp32 tensor as one tensor (one amax, one fp32
 * tensor scale). codes: [rows][K/2]; scales: [rows][K/16]; chose4: optional
 * [rows][K/16] flags. K must be a multiple of 16. mode as in nvfp4_block.
 */
int orc_quant_nvfp4_mode(const float *x, int64_t rows, int64_t K, int mode, uint8_t *codes,
                         uint8_t *scales, float *tensor_scale, uint8_t *chose4) {
    if (!x || !codes || !scales || !tensor_scale || rows < 0 || K <= 0 || K % 16) return ORC_EINVAL;
    if (mode < 0 || mode > 2) return ORC_EINVAL;
    init_tables();
    float amax = 0.0f;
    for (int64_t i = 0; i < rows * K; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float sg = orc_nvfp4_tensor_scale(amax);
    *tensor_scale = sg;
    int64_t nb = rows * (K / 16);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        int c4 = nvfp4_block(x + b * 16, sg, mode, codes + b * 8, scales + b);
        if (chose4) chose4[b] = (uint8_t)c4;
    }
    return ORC_OK;
}

/* The 4-vs-6 rule ([A] "TL;DR"). */
int orc_quant_nvfp4(const float *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales,
                    float *tensor_scale, uint8_t *chose4) {
    return orc_quant_nvfp4_mode(x, rows, K, 0, codes, scales, tensor_scale, chose4);
}

/* Same, for bf16 input (bit patterns); bf16 widens to fp32 exactly. */
static inline float bf16_value(uint16_t u) {
    uint32_t w = (uint32_t)u << 16;
    float f;
    memcpy(&f, &w, 4);
    return f;
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even: the 16 dropped bits are
 * compared with half an ulp of the kept part (inputs here are finite). */
static uint16_t bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    const uint32_t kept = u >> 16, dropped = u & 0xffffu;
    uint32_t r = kept;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) r = kept + 1u;
    return (uint16_t)r;
}

/* ------------------------------------------------------------------------- */
/* MXFP8 quantiser: E4M3 elements, E8M0 scale per 32 ([R] "Overview").        */
/* ------------------------------------------------------------------------- */

static void mxfp8_block(const float *x, uint8_t *codes32, uint8_t *scale) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    int sc = orc_e8m0_code_for_amax(amax);
    int se = sc - 127;
    for (int i = 0; i < 32; ++i) codes32[i] = (uint8_t)orc_e4m3_encode(ldexp((double)x[i], -se));
    *scale = (uint8_t)sc;
}

/* codes: [rows][K]; scales: [rows][K/32]. K must be a multiple of 32. */
int orc_quant_mxfp8(const float *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales) {
    if (!x || !codes || !scales || rows < 0 || K <= 0 || K % 32) return ORC_EINVAL;
    init_tables();
    int64_t nb = rows * (K / 32);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) mxfp8_block(x + b * 32, codes + b * 32, scales + b);
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* MXFP4 quantiser: E2M1 elements, E8M0 scale per 32 ([V] "Variants").        */
/* ------------------------------------------------------------------------- */

/* codes16: the block's 32 E2M1 codes, element 2i in the low nibble of byte i */
static void mxfp4_block(const float *x, uint8_t *codes16, uint8_t *scale) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    int sc = orc_mxfp4_scale_code(amax);
    int se = sc - 127;
    for (int i = 0; i < 16; ++i) {
        int lo = orc_e2m1_encode(ldexp((double)x[2 * i], -se));
        int hi = orc_e2m1_encode(ldexp((double)x[2 * i + 1], -se));
        codes16[i] = (uint8_t)(lo | (hi << 4));
    }
    *scale = (uint8_t)sc;
}

/* codes: [rows][K/2]; scales: [rows][K/32]. K must be a multiple of 32. */
int orc_quant_mxfp4(const float *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales) {
    if (!x || !codes || !scales || rows < 0 || K <= 0 || K % 32) return ORC_EINVAL;
    init_tables();
    int64_t nb = rows * (K / 32);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) mxfp4_block(x + b * 32, codes + b * 16, scales + b);
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* FP8 with one fp32 scale per row ([V] "Variants", variants.fp8: E4M3 with    */
/* dynamic per-token activation quantisation; weights: one scale per output   */
/* channel, i.e. per row of W [N][K]).                                        */
/* ------------------------------------------------------------------------- */

/* Row scale: fp32 amax / 448 (E4M3's largest value), or 1 for an all-zero row. */
float orc_fp8_row_scale(float amax) {
    return amax > 0.0f ? amax / 448.0f : 1.0f;
}

/* codes [rows][K]: E4M3 (nearest, ties to even, saturating, sign kept) of the fp32
 * quotient x / s_row; scales [rows] fp32. */
int orc_quant_fp8_rows(const float *x, int64_t rows, int64_t K, uint8_t *codes, float *scales) {
    if (!x || !codes || !scales || rows < 0 || K <= 0) return ORC_EINVAL;
    init_tables();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * K;
        float amax = 0.0f;
        for (int64_t i = 0; i < K; ++i) {
            float a = fabsf(xr[i]);
            if (a > amax) amax = a;
        }
        float s = orc_fp8_row_scale(amax);
        for (int64_t i = 0; i < K; ++i) {
            float q = xr[i] / s;
            codes[r * K + i] = (uint8_t)orc_e4m3_encode((double)q);
        }
        scales[r] = s;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Dequantisation (fp64).                                                     */
/* ------------------------------------------------------------------------- */

/* x_hat = e4m3(code) [* scale of its row if with_scale]. */
int orc_dequant_fp8_rows(const uint8_t *codes, const float *scales, int64_t rows, int64_t K, int with_scale,
                         double *out) {
    if (!codes || !out || (with_scale && !scales) || rows < 0 || K <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * K; ++i) {
        double v = orc_e4m3_value(codes[i]);
        out[i] = with_scale ? v * (double)scales[i / K] : v;
    }
    return ORC_OK;
}

/* x_hat = e2m1(code) * e4m3(scale) [* tensor_scale if with_tensor]. */
int orc_dequant_nvfp4(const uint8_t *codes, const uint8_t *scales, float tensor_scale, int64_t rows,
                      int64_t K, int with_tensor, double *out) {
    if (!codes || !scales || !out || K % 16) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * K; ++i) {
        int c = (codes[i / 2] >> ((i & 1) * 4)) & 15;
        double v = orc_e2m1_value(c) * orc_e4m3_value(scales[i / 16]);
        out[i] = with_tensor ? v * (double)tensor_scale : v;
    }
    return ORC_OK;
}

int orc_dequant_mxfp8(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, double *out) {
    if (!codes || !scales || !out || K % 32) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * K; ++i) out[i] = orc_e4m3_value(codes[i]) * orc_e8m0_value(scales[i / 32]);
    return ORC_OK;
}

/* x_hat = e2m1(code) * e8m0(scale) */
int orc_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, double *out) {
    if (!codes || !scales || !out || K % 32) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * K; ++i) {
        int c = (codes[i / 2] >> ((i & 1) * 4)) & 15;
        out[i] = orc_e2m1_value(c) * orc_e8m0_value(scales[i / 32]);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Weight quantisation over E experts (one tensor per expert per matrix).     */
/* ------------------------------------------------------------------------- */

/* fp32 [n] -> bf16 bit patterns [n], nearest, ties to even. */
int orc_round_bf16(const float *x, int64_t n, uint16_t *out) {
    if (n < 0 || (n && (!x || !out))) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(x[i]);
    return ORC_OK;
}

/* fmt 1 = NVFP4, 2 = MXFP8, 3 = MXFP4, 6 = FP8 per channel. w: bf16 [E][N][K].
 * tensor_scale: fp32 [E] (NVFP4) or fp32 [E][N], one per output channel (FP8); scales
 * unused by FP8 (may be NULL). */
int orc_quantize_weights(int fmt, int32_t E, int32_t N, int32_t K, const uint16_t *w, uint8_t *codes,
                         uint8_t *scales, float *tensor_scale) {
    if (!w || !codes || (!scales && fmt != 6) || E <= 0 || N <= 0 || K <= 0) return ORC_EINVAL;
    if ((fmt == 1 || fmt == 6) && !tensor_scale) return ORC_EINVAL;
    if (fmt == 1 && K % 16) return ORC_EINVAL;
    if ((fmt == 2 || fmt == 3) && K % 32) return ORC_EINVAL;
    if (fmt < 1 || (fmt > 3 && fmt != 6)) return ORC_EINVAL;
    int64_t per = (int64_t)N * K;
    float *buf = (float *)malloc(sizeof(float) * per);
    if (!buf) return ORC_ENOMEM;
    int rc = ORC_OK;
    for (int32_t e = 0; e < E && rc == ORC_OK; ++e) {
        const uint16_t *src = w + e * per;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < per; ++i) buf[i] = bf16_value(src[i]);
        if (fmt == 1)
            rc = orc_quant_nvfp4(buf, N, K, codes + e * per / 2, scales + e * per / 16, tensor_scale + e, NULL);
        else if (fmt == 2)
            rc = orc_quant_mxfp8(buf, N, K, codes + e * per, scales + e * per / 32);
        else if (fmt == 6) /* one scale per output channel (row) */
            rc = orc_quant_fp8_rows(buf, N, K, codes + e * per, tensor_scale + e * N);
        else
            rc = orc_quant_mxfp4(buf, N, K, codes + e * per / 2, scales + e * per / 32);
    }
    free(buf);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Router: softmax over E logits, top-k, renormalised weights.                */
/* ------------------------------------------------------------------------- */

/*
 * logits[t][e] = sum_{d ascending} h[t][d] * wr[e][d] in fp32 from +0 (each
 * bf16 x bf16 product is exact in fp32), plus bias[e] in fp32 if given.
 * The top-k experts are the k largest logits, ties to the lower index, in
 * that rank order; their weights are softmax over all E renormalised over the
 * k, i.e. exp(l_j - l_max) / sum_i exp(l_i - l_max) over the selected (fp64).
 */
int orc_route(int32_t T, int32_t D, int32_t E, int32_t k, const uint16_t *h, const uint16_t *wr,
              const float *bias, int32_t *idx, float *w, float *logits_out) {
    if (T < 0 || D <= 0 || E <= 0 || k <= 0 || k > E || (T > 0 && (!h || !wr || !idx || !w)))
        return ORC_EINVAL;
    int rc = ORC_OK;
#pragma omp parallel
    {
        float *lg = (float *)malloc(sizeof(float) * E);
        unsigned char *taken = (unsigned char *)malloc(E);
        if (!lg || !taken) {
#pragma omp atomic write
            rc = ORC_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int32_t t = 0; t < T; ++t) {
                for (int32_t e = 0; e < E; ++e) {
                    float acc = 0.0f;
                    for (int32_t d = 0; d < D; ++d)
                        acc = acc + bf16_value(h[(int64_t)t * D + d]) * bf16_value(wr[(int64_t)e * D + d]);
                    if (bias) acc = acc + bias[e];
                    lg[e] = acc;
                    if (logits_out) logits_out[(int64_t)t * E + e] = acc;
                    taken[e] = 0;
                }
                for (int32_t j = 0; j < k; ++j) {
                    int32_t best = -1;
                    for (int32_t e = 0; e < E; ++e) {
                        if (taken[e]) continue;
                        if (best < 0 || lg[e] > lg[best]) best = e; /* strict: lower index wins ties */
                    }
                    taken[best] = 1;
                    idx[(int64_t)t * k + j] = best;
                }
                double lmax = lg[idx[(int64_t)t * k]];
                double den = 0.0;
                for (int32_t j = 0; j < k; ++j) den += exp((double)lg[idx[(int64_t)t * k + j]] - lmax);
                for (int32_t j = 0; j < k; ++j)
                    w[(int64_t)t * k + j] = (float)(exp((double)lg[idx[(int64_t)t * k + j]] - lmax) / den);
            }
        }
        free(lg);
        free(taken);
    }
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Permutation: stable grouping of the local token-slots by expert.           */
/* ------------------------------------------------------------------------- */

/*
 * Slot s = t*k + j is local when idx[s] lies in [e_begin, e_end). The local
 * slots are ordered by expert, and by s within an expert. counts[e - e_begin]
 * = slots of expert e; offsets = exclusive prefix sum (n+1 entries);
 * sorted_slot[p] = the slot at position p. Returns the number of local slots.
 */
int64_t orc_permute(int32_t T, int32_t k, const int32_t *idx, int32_t e_begin, int32_t e_end,
                    int32_t *counts, int32_t *offsets, int32_t *sorted_slot) {
    if (T < 0 || k <= 0 || e_end <= e_begin || !counts || !offsets) return ORC_EINVAL;
    int32_t n = e_end - e_begin;
    for (int32_t e = 0; e < n; ++e) counts[e] = 0;
    for (int64_t s = 0; s < (int64_t)T * k; ++s) {
        int32_t e = idx[s];
        if (e >= e_begin && e < e_end) counts[e - e_begin]++;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < n; ++e) offsets[e + 1] = offsets[e] + counts[e];
    if (sorted_slot) {
        int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (n > 0 ? n : 1));
        if (!fill) return ORC_ENOMEM;
        for (int32_t e = 0; e < n; ++e) fill[e] = offsets[e];
        for (int64_t s = 0; s < (int64_t)T * k; ++s) {
            int32_t e = idx[s];
            if (e >= e_begin && e < e_end) sorted_slot[fill[e - e_begin]++] = (int32_t)s;
        }
        free(fill);
    }
    return offsets[n];
}

/* ------------------------------------------------------------------------- */
/* The MoE layer forward.                                                     */
/* ------------------------------------------------------------------------- */

typedef struct {
    int32_t fmt; /* 0 = unquantised bf16 masters (all fp64), 1 = NVFP4 W4A4, 2 = MXFP8 W8A8,
                    3 = MXFP4 W4A4, 4 = NVFP4 weights with bf16 activations (W4A16),
                    5 = bf16 experts: the bf16 masters with fp32 sums and a bf16 intermediate,
                    6 = FP8: E4M3 weights with a scale per output channel (gu_tscale [E][2F],
                        dn_tscale [E][D]) and E4M3 activations with a dynamic scale per row
                        (taps: a_tscale [T] and inter_tscale [S] hold the row scales) */
    int32_t T, D, F, E, k, e_begin, e_end;
    const uint16_t *h;  /* bf16 [T][D] */
    const int32_t *idx; /* [T][k] */
    const float *w;     /* [T][k] */
    /* fmt 0 and 5 */
    const uint16_t *gu_master; /* bf16 [E][2F][D]; rows [0,F) gate, [F,2F) up */
    const uint16_t *dn_master; /* bf16 [E][D][F] */
    /* fmt 1-4: canonical packed layout (see orc_quantize_weights; fmt 4 uses NVFP4's) */
    const uint8_t *gu_codes, *gu_scales;
    const float *gu_tscale;
    const uint8_t *dn_codes, *dn_scales;
    const float *dn_tscale;
    float *out; /* fp32 [T][D] */
    /* optional taps (NULL = skip); slot-indexed arrays are in sorted order */
    uint8_t *a_codes, *a_scales;
    float *a_tscale;
    float *inter; /* pre-quantisation SwiGLU output, fp32 [S][F] */
    uint8_t *inter_codes, *inter_scales; /* fmt 4: bf16 bit patterns [S][F] (2 bytes each), no scales */
    float *inter_tscale;
    float *y;  /* down projection per slot (before the gate weight), fp32 [S][D] */
    double *inter_abs; /* optional: sum_k |a_k w_k| of the gate (j < F) and up (j >= F)
                          accumulations, fp64 [S][2F] */
    /* optional: compute only these output tokens (others are left zero). The
       NVFP4 intermediate tensor scale still covers every local slot. */
    const int32_t *tok_list;
    int32_t n_tok;
} orc_moe_args;

/* SwiGLU: silu(g) * u = g * u / (1 + exp(-g)), evaluated in fp64 and rounded once to fp32. */
static float swiglu_f32(float g, float u) {
    return (float)((double)g * (double)u / (1.0 + exp(-(double)g)));
}

/* Weight row r of expert e for the given matrix, dequantised to fp64 WITHOUT
 * the NVFP4 tensor scale or the FP8 channel scale (those factors are applied to the
 * fp32 sum). */
static void weight_row(int fmt, const uint16_t *master, const uint8_t *codes, const uint8_t *scales,
                       int64_t row_index, int64_t K, double *out) {
    int64_t base = row_index * K;
    for (int64_t j = 0; j < K; ++j) {
        int64_t i = base + j;
        if (fmt == 0) {
            out[j] = bf16_value(master[i]);
        } else if (fmt == 1) {
            int c = (codes[i / 2] >> ((i & 1) * 4)) & 15;
            out[j] = orc_e2m1_value(c) * orc_e4m3_value(scales[i / 16]);
        } else if (fmt == 2) {
            out[j] = orc_e4m3_value(codes[i]) * orc_e8m0_value(scales[i / 32]);
        } else if (fmt == 6) { /* the channel scale is applied to the fp32 sum */
            out[j] = orc_e4m3_value(codes[i]);
        } else {
            int c = (codes[i / 2] >> ((i & 1) * 4)) & 15;
            out[j] = orc_e2m1_value(c) * orc_e8m0_value(scales[i / 32]);
        }
    }
}

/*
 * Forward of the MoE layer for the local experts [e_begin, e_end):
 *  1. quantise the hidden states once per token to the layer's format;
 *  2. for each local slot (t, j) routed to expert e: gate and up rows of
 *     A_t . W_gu[e]^T summed in fp64; NVFP4 multiplies the fp32-rounded sum by
 *     fl32(s_A * s_W) and rounds again; MXFP8 and MXFP4 round the sum to fp32;
 *  3. h = SwiGLU(gate, up) (fp64, rounded once to fp32);
 *  4. quantise h to the layer's format (NVFP4: one tensor = all local slots);
 *  5. y = h_hat . W_d[e]^T in fp64, scaled and rounded as in 2;
 *  6. out[t] = sum over the token's local slots, j ascending, of w[t][j] * y
 *     (fp64, rounded to fp32); tokens without local slots get zeros.
 * fmt 0 runs the same steps on the bf16 masters entirely in fp64 (no
 * quantisation and no intermediate fp32 rounding). fmt 4 (W4A16: NVFP4 weights
 * dequantised on the fly, activations kept in bf16; vLLM recipe
 * "thinkingmachines/Inkling-Small", section "Variants") skips step 1, multiplies the
 * fp32-rounded sums of 2 and 5 by the weight tensor scale alone, and in step 4 rounds
 * h to bf16 (nearest, ties to even). fmt 5 (bf16 experts, the checkpoint's BF16 variant
 * in the same section) runs fmt 4's steps on the bf16 masters: exact products, sums rounded
 * to fp32 with no scale, h rounded to bf16. fmt 6 (FP8 with dynamic per-token activation
 * scales, same recipe, variants.fp8) quantises h per token row and the intermediate per
 * slot row (scale = row max / 448), and multiplies the fp32-rounded sums of 2 and 5 by
 * fl32(row scale * the weight row's channel scale).
 */
int orc_moe_forward(const orc_moe_args *a) {
    if (!a || a->T < 0 || a->D <= 0 || a->F <= 0 || a->E <= 0 || a->k <= 0 || a->k > a->E) return ORC_EINVAL;
    if (a->e_begin < 0 || a->e_end > a->E || a->e_end <= a->e_begin) return ORC_EINVAL;
    if (a->fmt < 0 || a->fmt > 6) return ORC_EINVAL;
    const int fmt = a->fmt;
    const int wf = fmt == 4 ? 1 : (fmt == 5 ? 0 : fmt); /* weight format (0: the bf16 masters) */
    const int a16 = fmt == 4 || fmt == 5;               /* bf16 activations, bf16 intermediate */
    const int64_t T = a->T, D = a->D, F = a->F, k = a->k;
    if (wf == 1 && (D % 16 || F % 16)) return ORC_EINVAL;
    if ((fmt == 2 || fmt == 3) && (D % 32 || F % 32)) return ORC_EINVAL;
    if (T == 0) return ORC_OK;
    if (!a->h || !a->idx || !a->w || !a->out) return ORC_EINVAL;
    if (wf == 0 && (!a->gu_master || !a->dn_master)) return ORC_EINVAL;
    if (wf == 1 && (!a->gu_codes || !a->gu_scales || !a->gu_tscale || !a->dn_codes || !a->dn_scales || !a->dn_tscale))
        return ORC_EINVAL;
    if ((fmt == 2 || fmt == 3) && (!a->gu_codes || !a->gu_scales || !a->dn_codes || !a->dn_scales)) return ORC_EINVAL;
    if (fmt == 6 && (!a->gu_codes || !a->gu_tscale || !a->dn_codes || !a->dn_tscale)) return ORC_EINVAL;
    init_tables();

    const int32_t n_loc = a->e_end - a->e_begin;
    int rc = ORC_OK;
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * n_loc);
    int32_t *offs = (int32_t *)malloc(sizeof(int32_t) * (n_loc + 1));
    int32_t *sorted = (int32_t *)malloc(sizeof(int32_t) * (T * k + 1));
    unsigned char *want_tok = (unsigned char *)calloc((size_t)T, 1);
    double *ahat = (double *)malloc(sizeof(double) * T * D);
    int64_t *cidx = NULL, *cdn = NULL;
    double *gu_raw = NULL, *ihat = NULL, *y64 = NULL, *inter64 = NULL;
    float *inter = NULL, *a_rs = NULL, *i_rs = NULL; /* FP8 row scales of h and of the intermediate */
    if (!counts || !offs || !sorted || !want_tok || !ahat) { rc = ORC_ENOMEM; goto done; }
    const int64_t S = orc_permute(a->T, a->k, a->idx, a->e_begin, a->e_end, counts, offs, sorted);

    if (a->tok_list) {
        for (int32_t i = 0; i < a->n_tok; ++i)
            if (a->tok_list[i] >= 0 && a->tok_list[i] < T) want_tok[a->tok_list[i]] = 1;
    } else {
        memset(want_tok, 1, (size_t)T);
    }

    /* compact indices: slots whose gate_up is needed (all of them for NVFP4,
     * whose intermediate tensor scale covers every local slot), and slots
     * whose down projection is needed (those of the wanted tokens) */
    cidx = (int64_t *)malloc(sizeof(int64_t) * (S + 1));
    cdn = (int64_t *)malloc(sizeof(int64_t) * (S + 1));
    if (!cidx || !cdn) { rc = ORC_ENOMEM; goto done; }
    int64_t ngu = 0, ndn = 0;
    for (int64_t p = 0; p < S; ++p) {
        int wanted = want_tok[sorted[p] / k];
        cidx[p] = (fmt == 1 || wanted) ? ngu++ : -1;
        cdn[p] = wanted ? ndn++ : -1;
    }

    /* 1. input activations, quantised once per token ([A] "NVFP4 and MXFP8 experts") */
    float a_ts = 1.0f;
    {
        float *hf = (float *)malloc(sizeof(float) * T * D);
        if (!hf) { rc = ORC_ENOMEM; goto done; }
        for (int64_t i = 0; i < T * D; ++i) hf[i] = bf16_value(a->h[i]);
        if (fmt == 0 || a16) {
            for (int64_t i = 0; i < T * D; ++i) ahat[i] = hf[i];
        } else if (fmt == 6) {
            uint8_t *ac = (uint8_t *)malloc(T * D);
            a_rs = (float *)malloc(sizeof(float) * T);
            if (!ac || !a_rs) { free(hf); free(ac); rc = ORC_ENOMEM; goto done; }
            orc_quant_fp8_rows(hf, T, D, ac, a_rs);
            orc_dequant_fp8_rows(ac, a_rs, T, D, 0, ahat);
            if (a->a_codes) memcpy(a->a_codes, ac, T * D);
            if (a->a_tscale) memcpy(a->a_tscale, a_rs, sizeof(float) * T);
            free(ac);
        } else {
            int64_t nc = fmt == 2 ? T * D : T * D / 2, ns = fmt == 1 ? T * D / 16 : T * D / 32;
            uint8_t *ac = (uint8_t *)malloc(nc), *as = (uint8_t *)malloc(ns);
            if (!ac || !as) { free(hf); free(ac); free(as); rc = ORC_ENOMEM; goto done; }
            if (fmt == 1) {
                orc_quant_nvfp4(hf, T, D, ac, as, &a_ts, NULL);
                orc_dequant_nvfp4(ac, as, a_ts, T, D, 0, ahat);
            } else if (fmt == 2) {
                orc_quant_mxfp8(hf, T, D, ac, as);
                orc_dequant_mxfp8(ac, as, T, D, ahat);
            } else {
                orc_quant_mxfp4(hf, T, D, ac, as);
                orc_dequant_mxfp4(ac, as, T, D, ahat);
            }
            if (a->a_codes) memcpy(a->a_codes, ac, nc);
            if (a->a_scales) memcpy(a->a_scales, as, ns);
            if (a->a_tscale) *a->a_tscale = a_ts;
            free(ac);
            free(as);
        }
        free(hf);
    }

    /* 2. gate_up sums in fp64: gu_raw[c][r], r in [0, 2F) */
    gu_raw = (double *)malloc(sizeof(double) * (ngu > 0 ? ngu : 1) * 2 * F);
    if (!gu_raw) { rc = ORC_ENOMEM; goto done; }
    {
        const int64_t nrows = 2 * F;
        int fail = 0;
#pragma omp parallel
        {
            double *wrow = (double *)malloc(sizeof(double) * D);
            if (!wrow) {
#pragma omp atomic write
                fail = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t it = 0; it < (int64_t)n_loc * nrows; ++it) {
                    int32_t el = (int32_t)(it / nrows);
                    int64_t r = it % nrows;
                    int any = 0;
                    for (int64_t p = offs[el]; p < offs[el + 1]; ++p) any |= cidx[p] >= 0;
                    if (!any) continue;
                    weight_row(wf, a->gu_master, a->gu_codes, a->gu_scales,
                               (int64_t)(a->e_begin + el) * nrows + r, D, wrow);
                    for (int64_t p = offs[el]; p < offs[el + 1]; ++p) {
                        if (cidx[p] < 0) continue;
                        const double *arow = ahat + (int64_t)(sorted[p] / k) * D;
                        double s = 0.0, sa = 0.0;
                        for (int64_t d = 0; d < D; ++d) {
                            double pr = arow[d] * wrow[d];
                            s += pr;
                            sa += fabs(pr);
                        }
                        gu_raw[cidx[p] * nrows + r] = s;
                        if (a->inter_abs) a->inter_abs[p * nrows + r] = sa;
                    }
                }
            }
            free(wrow);
        }
        if (fail) { rc = ORC_ENOMEM; goto done; }
    }

    /* 3. SwiGLU: inter (fp32) or inter64 (fmt 0) in compact gate_up order */
    if (fmt == 0) {
        inter64 = (double *)malloc(sizeof(double) * (ngu > 0 ? ngu : 1) * F);
        if (!inter64) { rc = ORC_ENOMEM; goto done; }
    } else {
        inter = (float *)malloc(sizeof(float) * (ngu > 0 ? ngu : 1) * F);
        if (!inter) { rc = ORC_ENOMEM; goto done; }
    }
    for (int64_t p = 0; p < S; ++p) {
        int64_t c = cidx[p];
        if (c < 0) continue;
        int32_t e = sorted[p] >= 0 ? a->idx[sorted[p]] : 0;
        float sc = fmt == 1 ? a_ts * a->gu_tscale[e] : (fmt == 4 ? a->gu_tscale[e] : 1.0f);
        for (int64_t f = 0; f < F; ++f) {
            double gr = gu_raw[c * 2 * F + f], ur = gu_raw[c * 2 * F + F + f];
            if (fmt == 0) {
                inter64[c * F + f] = gr * ur / (1.0 + exp(-gr));
            } else {
                float g = (float)gr, u = (float)ur;
                if (wf == 1) {
                    g = g * sc;
                    u = u * sc;
                } else if (fmt == 6) { /* token scale times the gate / up channel scale */
                    const float st = a_rs[sorted[p] / k];
                    g = g * (st * a->gu_tscale[(int64_t)e * 2 * F + f]);
                    u = u * (st * a->gu_tscale[(int64_t)e * 2 * F + F + f]);
                }
                float hv = swiglu_f32(g, u);
                inter[c * F + f] = hv;
                if (a->inter) a->inter[p * F + f] = hv;
            }
        }
    }

    /* 4. intermediate quantisation to the layer's format -> ihat (fp64, no tensor scale) */
    float i_ts = 1.0f;
    ihat = (double *)malloc(sizeof(double) * (ngu > 0 ? ngu : 1) * F);
    if (!ihat) { rc = ORC_ENOMEM; goto done; }
    if (fmt == 0) {
        memcpy(ihat, inter64, sizeof(double) * ngu * F);
    } else if (a16) {
        for (int64_t p = 0; p < S; ++p) {
            int64_t c = cidx[p];
            if (c < 0) continue;
            for (int64_t f = 0; f < F; ++f) {
                uint16_t b = bf16_rne(inter[c * F + f]);
                ihat[c * F + f] = bf16_value(b);
                if (a->inter_codes) memcpy(a->inter_codes + 2 * (p * F + f), &b, 2);
            }
        }
    } else if (fmt == 1) {
        /* every local slot is in the compact set, in sorted order (cidx[p] == p) */
        uint8_t *ic = (uint8_t *)malloc(S * F / 2 + 1), *is = (uint8_t *)malloc(S * F / 16 + 1);
        if (!ic || !is) { free(ic); free(is); rc = ORC_ENOMEM; goto done; }
        orc_quant_nvfp4(inter, S, F, ic, is, &i_ts, NULL);
        orc_dequant_nvfp4(ic, is, i_ts, S, F, 0, ihat);
        if (a->inter_codes) memcpy(a->inter_codes, ic, S * F / 2);
        if (a->inter_scales) memcpy(a->inter_scales, is, S * F / 16);
        if (a->inter_tscale) *a->inter_tscale = i_ts;
        free(ic);
        free(is);
    } else if (fmt == 6) {
        /* every local slot's row with its own dynamic scale */
        uint8_t *ic = (uint8_t *)malloc(F);
        i_rs = (float *)malloc(sizeof(float) * (S > 0 ? S : 1));
        if (!ic || !i_rs) { free(ic); rc = ORC_ENOMEM; goto done; }
        for (int64_t p = 0; p < S; ++p) {
            int64_t c = cidx[p];
            if (c < 0) continue;
            orc_quant_fp8_rows(inter + c * F, 1, F, ic, i_rs + p);
            orc_dequant_fp8_rows(ic, i_rs + p, 1, F, 0, ihat + c * F);
            if (a->inter_codes) memcpy(a->inter_codes + p * F, ic, F);
            if (a->inter_tscale) a->inter_tscale[p] = i_rs[p];
        }
        free(ic);
    } else {
        /* MXFP8 [S][F] codes, MXFP4 [S][F/2]; both [S][F/32] scales */
        const int64_t cb = fmt == 2 ? F : F / 2;
        uint8_t *ic = (uint8_t *)malloc(cb), *is = (uint8_t *)malloc(F / 32);
        if (!ic || !is) { free(ic); free(is); rc = ORC_ENOMEM; goto done; }
        for (int64_t p = 0; p < S; ++p) {
            int64_t c = cidx[p];
            if (c < 0) continue;
            if (fmt == 2) {
                orc_quant_mxfp8(inter + c * F, 1, F, ic, is);
                orc_dequant_mxfp8(ic, is, 1, F, ihat + c * F);
            } else {
                orc_quant_mxfp4(inter + c * F, 1, F, ic, is);
                orc_dequant_mxfp4(ic, is, 1, F, ihat + c * F);
            }
            if (a->inter_codes) memcpy(a->inter_codes + p * cb, ic, cb);
            if (a->inter_scales) memcpy(a->inter_scales + p * F / 32, is, F / 32);
        }
        free(ic);
        free(is);
    }

    /* 5. down projection for the wanted slots: y64[cdn][n] */
    y64 = (double *)malloc(sizeof(double) * (ndn > 0 ? ndn : 1) * D);
    if (!y64) { rc = ORC_ENOMEM; goto done; }
    {
        int fail = 0;
#pragma omp parallel
        {
            double *wrow = (double *)malloc(sizeof(double) * F);
            if (!wrow) {
#pragma omp atomic write
                fail = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t it = 0; it < (int64_t)n_loc * D; ++it) {
                    int32_t el = (int32_t)(it / D);
                    int64_t n = it % D;
                    int any = 0;
                    for (int64_t p = offs[el]; p < offs[el + 1]; ++p) any |= cdn[p] >= 0;
                    if (!any) continue;
                    int32_t e = a->e_begin + el;
                    weight_row(wf, a->dn_master, a->dn_codes, a->dn_scales, (int64_t)e * D + n, F, wrow);
                    float sc = fmt == 1 ? i_ts * a->dn_tscale[e] : (fmt == 4 ? a->dn_tscale[e] : 1.0f);
                    for (int64_t p = offs[el]; p < offs[el + 1]; ++p) {
                        if (cdn[p] < 0) continue;
                        const double *irow = ihat + cidx[p] * F;
                        double s = 0.0;
                        for (int64_t f = 0; f < F; ++f) s += irow[f] * wrow[f];
                        double yv;
                        if (fmt == 0) yv = s;
                        else if (wf == 1) yv = (float)((float)s * sc);
                        else if (fmt == 6) yv = (float)((float)s * (i_rs[p] * a->dn_tscale[(int64_t)e * D + n]));
                        else yv = (float)s;
                        y64[cdn[p] * D + n] = yv;
                        if (a->y) a->y[p * D + n] = (float)yv;
                    }
                }
            }
            free(wrow);
        }
        if (fail) { rc = ORC_ENOMEM; goto done; }
    }

    /* 6. combine: gather each token's local slots in j order */
    {
        int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * T * k);
        if (!pos) { rc = ORC_ENOMEM; goto done; }
        for (int64_t s = 0; s < T * k; ++s) pos[s] = -1;
        for (int64_t p = 0; p < S; ++p) pos[sorted[p]] = p;
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            float *o = a->out + t * D;
            if (!want_tok[t]) continue;
            for (int64_t n = 0; n < D; ++n) {
                double acc = 0.0;
                for (int64_t j = 0; j < k; ++j) {
                    int64_t p = pos[t * k + j];
                    if (p < 0) continue;
                    acc += (double)a->w[t * k + j] * y64[cdn[p] * D + n];
                }
                o[n] = (float)acc;
            }
        }
        for (int64_t t = 0; t < T; ++t)
            if (!want_tok[t]) memset(a->out + t * D, 0, sizeof(float) * D);
        free(pos);
    }

done:
    free(counts); free(offs); free(sorted); free(want_tok); free(ahat);
    free(cidx); free(cdn); free(gu_raw); free(ihat); free(y64); free(inter64); free(inter);
    free(a_rs); free(i_rs);
    return rc;
}

/*
 * Steps 5 and 6 of the forward alone, from given intermediate codes: for each local
 * slot p (sorted order as orc_permute gives it), y = dequant(intermediate row p) . W_d[e]^T
 * summed in fp64 and rounded and scaled exactly as in orc_moe_forward, then
 * out[t] = sum over the token's local slots, j ascending, of w[t][j] * y (fp64, rounded
 * to fp32). Used to check a down projection and combine on another implementation's
 * intermediate codes. i_codes / i_scales: [S][F/2] and [S][F/16] (NVFP4, tensor scale
 * i_ts), [S][F] and [S][F/32] (MXFP8), [S][F/2] and [S][F/32] (MXFP4), or bf16 bit
 * patterns [S][F] (2 bytes each) and no scales (W4A16, fmt 4, and bf16 experts, fmt 5,
 * whose dn_codes are the bf16 masters [E][D][F] and dn_scales may be NULL), or E4M3 codes
 * [S][F] with fp32 row scales i_row_scales [S] (FP8, fmt 6: dn_tscale holds the channel
 * scales [E][D]; dn_scales unused).
 */
int orc_down_combine(int32_t fmt, int32_t T, int32_t D, int32_t F, int32_t E, int32_t k, int32_t e_begin,
                     int32_t e_end, const int32_t *idx, const float *w, const uint8_t *i_codes,
                     const uint8_t *i_scales, float i_ts, const uint8_t *dn_codes, const uint8_t *dn_scales,
                     const float *dn_tscale, const float *i_row_scales, float *out) {
    if (fmt < 1 || fmt > 6) return ORC_EINVAL;
    const int wf = fmt == 4 ? 1 : (fmt == 5 ? 0 : fmt);
    if (T < 0 || D <= 0 || F <= 0 || E <= 0 || k <= 0 || e_begin < 0 || e_end > E || e_end <= e_begin) return ORC_EINVAL;
    if (T == 0) return ORC_OK;
    if (!idx || !w || !i_codes || (fmt < 4 && !i_scales) || !dn_codes || (wf != 0 && wf != 6 && !dn_scales) ||
        !out || ((wf == 1 || wf == 6) && !dn_tscale) || (fmt == 6 && !i_row_scales))
        return ORC_EINVAL;
    init_tables();
    const int32_t n_loc = e_end - e_begin;
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * n_loc);
    int32_t *offs = (int32_t *)malloc(sizeof(int32_t) * (n_loc + 1));
    int32_t *sorted = (int32_t *)malloc(sizeof(int32_t) * ((int64_t)T * k + 1));
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (int64_t)T * k);
    double *ihat = NULL, *y64 = NULL;
    int rc = ORC_OK;
    if (!counts || !offs || !sorted || !pos) { rc = ORC_ENOMEM; goto done; }
    const int64_t S = orc_permute(T, k, idx, e_begin, e_end, counts, offs, sorted);
    ihat = (double *)malloc(sizeof(double) * (S > 0 ? S : 1) * F);
    y64 = (double *)malloc(sizeof(double) * (S > 0 ? S : 1) * D);
    if (!ihat || !y64) { rc = ORC_ENOMEM; goto done; }
    if (fmt == 1) orc_dequant_nvfp4(i_codes, i_scales, i_ts, S, F, 0, ihat);
    else if (fmt == 2) orc_dequant_mxfp8(i_codes, i_scales, S, F, ihat);
    else if (fmt == 3) orc_dequant_mxfp4(i_codes, i_scales, S, F, ihat);
    else if (fmt == 6) orc_dequant_fp8_rows(i_codes, i_row_scales, S, F, 0, ihat);
    else /* fmt 4 and 5: bf16 */
        for (int64_t i = 0; i < S * F; ++i) {
            uint16_t b;
            memcpy(&b, i_codes + 2 * i, 2);
            ihat[i] = bf16_value(b);
        }
    {
        int fail = 0;
#pragma omp parallel
        {
            double *wrow = (double *)malloc(sizeof(double) * F);
            if (!wrow) {
#pragma omp atomic write
                fail = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t it = 0; it < (int64_t)n_loc * D; ++it) {
                    int32_t el = (int32_t)(it / D);
                    int64_t n = it % D;
                    if (offs[el] == offs[el + 1]) continue;
                    int32_t e = e_begin + el;
                    weight_row(wf, (const uint16_t *)dn_codes, dn_codes, dn_scales, (int64_t)e * D + n, F, wrow);
                    float sc = fmt == 1 ? i_ts * dn_tscale[e] : (fmt == 4 ? dn_tscale[e] : 1.0f);
                    for (int64_t p = offs[el]; p < offs[el + 1]; ++p) {
                        const double *irow = ihat + p * F;
                        double s = 0.0;
                        for (int64_t f = 0; f < F; ++f) s += irow[f] * wrow[f];
                        if (fmt == 6)
                            y64[p * D + n] = (double)(float)((float)s * (i_row_scales[p] * dn_tscale[(int64_t)e * D + n]));
                        else
                            y64[p * D + n] = wf == 1 ? (double)(float)((float)s * sc) : (double)(float)s;
                    }
                }
            }
            free(wrow);
        }
        if (fail) { rc = ORC_ENOMEM; goto done; }
    }
    for (int64_t s = 0; s < (int64_t)T * k; ++s) pos[s] = -1;
    for (int64_t p = 0; p < S; ++p) pos[sorted[p]] = p;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < D; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                int64_t p = pos[t * k + j];
                if (p < 0) continue;
                acc += (double)w[t * k + j] * y64[p * D + n];
            }
            out[t * D + n] = (float)acc;
        }
    }
done:
    free(counts); free(offs); free(sorted); free(pos); free(ihat); free(y64);
    return rc;
}
