/*
 * moe.h - C ABI of the block-scaled routed-expert MoE layer for AMD MI355X (gfx950).
 *
 * The layer (vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview";
 * AI Primer "Thinking Machines releases Inkling 2 Small weights under Apache 2.0",
 * section "NVFP4 and MXFP8 experts"): every token is sent to 8 of 384 routed experts,
 * there is no shared expert, expert weights are NVFP4 (layers 0-39) or MXFP8 (layers
 * 40-47), and the expert activations are quantised to the layer's weight format.
 * The pages fix neither the gate, the expert MLP nor the bit layouts; the readings
 * used here are: softmax-then-top-8 gate, SwiGLU experts (gate_up [2F, D] with rows
 * [0, F) = gate and [F, 2F) = up, down [D, F]), NVFP4 = E2M1 codes + one E4M3 scale
 * per 16 values + an fp32 tensor scale amax / (6 * 448), with each 16-block scaled
 * so that its maximum maps to 6 or to 4, whichever gives the lower squared error
 * (AI Primer, section "TL;DR"), and MXFP8 = E4M3 codes + one E8M0 scale
 * 2^(floor(log2 amax) - 8) per 32 values.
 *
 * Conventions for every call:
 *  - All pointers are DEVICE pointers unless stated otherwise. The caller allocates
 *    and frees every buffer; the library allocates no device memory, holds no
 *    per-call global state and may be called concurrently on different streams
 *    with different buffers.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every
 *    call only enqueues work on it and returns; nothing synchronises the host.
 *  - Arguments are validated on the host before anything is enqueued; an invalid
 *    call returns a negative status and enqueues nothing. Faults inside kernels
 *    (for example from a bad pointer) surface at the caller's next synchronisation.
 *  - NaN or infinite inputs are outside the contract (results unspecified).
 *  - Device pointers must be 16-byte aligned (MOE_ERR_ALIGNMENT otherwise).
 */
#ifndef BLOCK_SCALED_MOE_H
#define BLOCK_SCALED_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 8

/* Status codes (0 = success). */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, bad size, bad range            */
#define MOE_ERR_UNSUPPORTED (-2) /* valid layer, but a shape this build rejects  */
#define MOE_ERR_ALIGNMENT (-3)   /* a device pointer is not 16-byte aligned      */
#define MOE_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required   */
#define MOE_ERR_HIP (-5)         /* a HIP launch failed                          */

/* Expert formats (recipe "Overview": NVFP4 in layers 0-39, MXFP8 in 40-47; MXFP4 is
 * the OCP MXFP4 W4A4 variant for AMD Instinct in the vLLM recipe
 * "thinkingmachines/Inkling-Small", section "Variants"; W4A16 is the NVFP4 checkpoint
 * run with bf16 activations, its weights dequantised on the fly, same section).
 * MOE_FMT_W4A16 is a moe_forward format only: its packed weights are MOE_FMT_NVFP4.
 * MOE_FMT_BF16 is the checkpoint's BF16 variant (same section): bf16 weights and
 * activations, fp32 accumulation, the SwiGLU output rounded to bf16.
 * MOE_FMT_FP8 is the FP8 variant of the same recipe (E4M3 with dynamic per-token
 * activation quantisation), read here as: E4M3 weights with one fp32 scale per output
 * channel, hidden states and the SwiGLU output E4M3 with one fp32 scale per row computed
 * at run time; every scale is fl32(max |row| / 448), 1 for an all-zero row. */
#define MOE_FMT_NVFP4 1
#define MOE_FMT_MXFP8 2
#define MOE_FMT_MXFP4 3
#define MOE_FMT_W4A16 4
#define MOE_FMT_BF16 5
#define MOE_FMT_FP8 6

/*
 * Packed expert weights of one matrix kind for E experts, each logically [N][K]
 * (K is the reduction dimension; N % 32 == 0, K % 64 == 0), stored per expert in a
 * tiled byte layout: the matrix is cut into 32-row x 64-column blocks kept in
 * block-row-major order ([N/32][K/64]); a block holds its 32 rows one after another,
 * each row with the codes of its 64 columns; the scales use the same block order.
 *   NVFP4: codes  u8 [E][N/32][K/64][32][32] E2M1, element 2i in the low nibble of byte i
 *          scales u8 [E][N/32][K/64][32][4]  E4M3 (OCP "FN": bias 7, max 448, no inf),
 *                                            one per 16 columns
 *          tensor_scale fp32 [E]  one per expert and matrix (amax / 2688, or 1)
 *   MXFP8: codes  u8 [E][N/32][K/64][4][32][16] E4M3: the block's 32 rows for columns
 *          0-15, then 16-31, 32-47, 48-63
 *          scales u8 [E][N/32][K/64][32][2]  E8M0 (2^(c - 127)), one per 32 columns
 *          tensor_scale unused (may be NULL)
 *   MXFP4: codes  u8 [E][N/32][K/64][2][32][16] E2M1, element 2i in the low nibble of
 *          byte i: the block's 32 rows for columns 0-31, then for columns 32-63
 *          scales u8 [E][N/32][K/64][2][32]  E8M0, one per 32 columns, same order
 *   BF16:  codes  u8 [E][N/32][K/64][2][32][64] bf16 values, the two 32-column halves
 *          of a block apart (column 32h + c at bytes 2c, 2c+1 of half h)
 *          scales, tensor_scale unused (may be NULL)
 *   FP8:   codes  u8 [E][N/32][K/64][4][32][16] E4M3, MXFP8's order
 *          scales unused (may be NULL)
 *          tensor_scale fp32 [E][N]  one per output channel (row): max |row| / 448, or 1
 * Sizes are those of the row-major arrays ([E][N][K/2] (NVFP4, MXFP4) / [E][N][K]
 * (MXFP8) codes, [E][N][K/16] (NVFP4) / [E][N][K/32] (MXFP8, MXFP4) scales); only the
 * order differs. The tiling lets one wave of the
 * expert GEMMs load a 32-row weight subtile's codes for 64 columns as a single
 * contiguous 1 KiB (NVFP4) or 2 KiB (MXFP8) run, each load instruction reading whole
 * cache lines; MXFP4's half-split order gives the scaled FP4 MFMA's 64 lanes (32 rows x
 * two 32-column halves) one contiguous 1 KiB.
 */
typedef struct moe_packed {
    int32_t fmt;
    int32_t E, N, K;
    uint8_t *codes;
    uint8_t *scales;
    float *tensor_scale;
} moe_packed;

/* Expert weights already quantised, in plain row-major arrays (a checkpoint's own
 * layout), one matrix kind [N][K] per expert for E experts:
 *   NVFP4: codes [E][N][K/2] E2M1, element 2i in the low nibble of byte i;
 *          scales [E][N][K/16] E4M3; tensor_scale fp32 [E]
 *   MXFP8: codes [E][N][K] E4M3; scales [E][N][K/32] E8M0; tensor_scale NULL
 *   MXFP4: codes [E][N][K/2] E2M1 (as NVFP4); scales [E][N][K/32] E8M0
 *   BF16:  codes [E][N][K] bf16 values (2 bytes each); scales, tensor_scale NULL
 *   FP8:   codes [E][N][K] E4M3; scales NULL; tensor_scale fp32 [E][N] channel scales */
typedef struct moe_rowmajor {
    int32_t fmt;
    int32_t E, N, K;
    const uint8_t *codes;
    const uint8_t *scales;
    const float *tensor_scale;
} moe_rowmajor;

/* Optional debug outputs of moe_forward (each pointer NULL = not written).
 * S = number of local token-slots (known on the device only; read offsets[n_loc]).
 * Slot-indexed arrays are in sorted (expert-grouped) order, sized for S <= T*top_k. */
typedef struct moe_taps {
    int32_t *counts;       /* [n_loc] slots per local expert                        */
    int32_t *offsets;      /* [n_loc + 1] exclusive prefix sum of counts            */
    int32_t *sorted_slot;  /* [T*top_k] slot id t*top_k + j at each sorted position  */
    uint8_t *a_codes;      /* hidden-state codes [T][D/2] (NVFP4, MXFP4) or [T][D]
                              (MXFP8, FP8); W4A16 writes neither these nor a_scales */
    uint8_t *a_scales;     /* [T][D/16] E4M3 (NVFP4) or [T][D/32] E8M0 (MX formats);
                              FP8 writes none                                      */
    float *a_tscale;       /* [1] NVFP4 hidden-state tensor scale; FP8: [T] row scales */
    float *inter;          /* [T*top_k][F] fp32 SwiGLU output before quantisation   */
    uint8_t *inter_codes;  /* [T*top_k][F/2] (NVFP4, MXFP4) or [T*top_k][F] (MXFP8,
                              FP8); W4A16: bf16 bit patterns [T*top_k][F], 2 bytes */
    uint8_t *inter_scales; /* [T*top_k][F/16] (NVFP4) or [T*top_k][F/32]; FP8: none  */
    float *inter_tscale;   /* [1] NVFP4 intermediate tensor scale; FP8: [T*top_k] row
                              scales in sorted order                               */
    float *y;              /* [T*top_k][D] fp32 down projection per slot (unweighted) */
} moe_taps;

/* moe_forward flags.
 * MOE_FLAG_EXACT_SUMS - MXFP8 layers: run the expert GEMMs on the codes expanded exactly
 *   to bf16 (the bf16 MFMA, fp32 sums with sequential-chain accuracy, about 2e-8 of the
 *   sum of |products| over K = 4096) instead of the gfx950 scaled FP8 MFMA on the codes
 *   and E8M0 scales as stored (twice the multiply rate; its sums are within about 2e-6 of
 *   the sum of |products|, so intermediate codes on a rounding boundary take the
 *   neighbouring code about 100 times as often). FP8 layers run on the scaled FP8 MFMA
 *   only and reject the flag (MOE_ERR_UNSUPPORTED). Other formats ignore it. */
#define MOE_FLAG_EXACT_SUMS 1u

/* Stage boundaries at which moe_forward records caller-created events (timing). */
#define MOE_EV_BEGIN 0        /* before the first kernel of the call          */
#define MOE_EV_GATE_UP 1      /* just before the gate_up GEMM                 */
#define MOE_EV_GATE_UP_END 2  /* just after the gate_up GEMM                  */
#define MOE_EV_DOWN 3         /* just before the down GEMM                    */
#define MOE_EV_DOWN_END 4     /* just after the down GEMM                     */
#define MOE_EV_END 5          /* after the last kernel (the combine)          */
#define MOE_N_EVENTS 6

/* Arguments of moe_forward. */
typedef struct moe_forward_args {
    int32_t fmt;              /* MOE_FMT_NVFP4, _MXFP8, _MXFP4, _W4A16, _BF16 or _FP8   */
    int32_t T, D, F, E;       /* tokens, d_model, d_ff, routed experts                  */
    int32_t top_k;            /* experts per token (8)                                  */
    int32_t e_begin, e_end;   /* local expert range [e_begin, e_end) computed here      */
    const uint16_t *h;        /* bf16 hidden states [T][D]                              */
    const float *h_amax;      /* NVFP4: max |h| as written by moe_route, or NULL        */
    const int32_t *topk_idx;  /* [T][top_k] experts per token, distinct within a row    */
    const float *topk_w;      /* [T][top_k] gate weights                                */
    moe_packed gate_up;       /* N = 2F, K = D                                          */
    moe_packed down;          /* N = D,  K = F                                          */
    float *out;               /* fp32 [T][D]; tokens without a local slot get zeros     */
    void *workspace;          /* device scratch of moe_forward_workspace_bytes() bytes  */
    size_t workspace_bytes;
    const moe_taps *taps;     /* host pointer to a moe_taps, or NULL                    */
    void *const *events;      /* NULL, or a host array of MOE_N_EVENTS hipEvent_t that are
                                 recorded on the stream at the MOE_EV_* boundaries      */
    uint32_t flags;           /* MOE_FLAG_* (0: the default routes)                     */
} moe_forward_args;

/* What moe_forward runs for given arguments (host only, from the size fields, fmt and
 * flags): the kernel family of each GEMM ("mx_gemm_kernel", "tile_gemm_kernel",
 * "stream_gemm_kernel", "grouped_gemm_kernel"; static strings), rows per M-tile and the
 * workspace size. */
typedef struct moe_plan_info {
    const char *gate_up_kernel;
    const char *down_kernel;
    int32_t m_tile_rows;
    size_t workspace_bytes;
} moe_plan_info;

/* ABI version (MOE_ABI_VERSION) and a static description of a status code. */
int32_t moe_abi_version(void);
const char *moe_status_string(int32_t status);

/*
 * Quantise bf16 expert weights w [E][N][K] into `out` (fmt, E, N, K and the three
 * buffers set by the caller). NVFP4 (AI Primer, "TL;DR"): per expert, tensor scale
 * s = amax/2688 (1 if the expert is all zero); per 16-block, r = amax_b / s, scale
 * candidates E4M3(r/6) and E4M3(r/4), codes E2M1(x / (E4M3 * s)), keep the candidate
 * with the smaller fp32 squared error (ties keep r/6). MXFP8: per 32-block, E8M0
 * exponent floor(log2 amax_b) - 8, codes E4M3(x * 2^-exponent). MXFP4: per 32-block,
 * E8M0 exponent floor(log2 amax_b) - 2, codes E2M1(x * 2^-exponent). FP8: per output
 * channel (row), scale s = fl32(amax_row / 448) (1 for an all-zero row) into
 * tensor_scale[e][n], codes E4M3(fl32(x / s)). All roundings are IEEE
 * round-to-nearest-even with saturation to the format's largest finite value.
 * N must be a multiple of 32 and K of 64 (the tiled layout above).
 */
int32_t moe_quantize_weights(const uint16_t *w, moe_packed *out, void *stream);

/*
 * Pack pre-quantised row-major weights `in` (a checkpoint in the format's plain layout,
 * vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview": the native NVFP4 /
 * MXFP8 checkpoint) into the tiled layout of `out` (fmt, E, N, K equal to in's; buffers
 * set by the caller): a pure reordering of the code and scale bytes, the tensor scales
 * copied. The bytes moe_quantize_weights writes for bf16 masters are the packing of the
 * row-major quantisation of the same masters (FP8: codes reordered, the E*N channel
 * scales copied). N % 32 == 0 and K % 64 == 0; in->codes and out's code and scale
 * buffers 16-byte aligned (MOE_ERR_ALIGNMENT), tensor scales 4-byte aligned. `in` and
 * `out` must not overlap.
 */
int32_t moe_pack_weights(const moe_rowmajor *in, moe_packed *out, void *stream);

/*
 * Router (softmax-then-top-k gate, recipe "Overview": 8 of 384 experts per token):
 *   logits[t][e] = sum over d ascending of h[t][d] * wr[e][d], accumulated in fp32
 *                  from +0 (each bf16 product is exact in fp32), plus bias[e] if given;
 *   topk_idx[t]  = the top_k largest logits, ties to the lower expert index, in rank
 *                  order;
 *   topk_w[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected (fp64,
 *                  rounded to fp32): the softmax over all E renormalised over the top_k.
 * h: bf16 [T][D]; wr: bf16 [E][D]; bias: fp32 [E] or NULL; logits: fp32 [T][E] or NULL
 * (if given, receives every logit above); h_amax: fp32 [1] or NULL (if given, receives
 * max |h| over all of h, for moe_forward's NVFP4 tensor scale). From 512 tokens on,
 * the top_k is found by screening MFMA-computed logits with a rigorous error bound and
 * recomputing the surviving candidates exactly, which gives the same indices and
 * weights. workspace: device scratch of at least moe_route_workspace_bytes(T, D, E)
 * bytes, caller-owned, contents undefined afterwards.
 * Requires 1 <= top_k <= 8, top_k <= E <= 1024, D % 64 == 0 (else
 * MOE_ERR_UNSUPPORTED). T = 0 is a no-op.
 */
size_t moe_route_workspace_bytes(int32_t T, int32_t D, int32_t E);
int32_t moe_route(int32_t T, int32_t D, int32_t E, int32_t top_k, const uint16_t *h,
                  const uint16_t *wr, const float *bias, float *logits, int32_t *topk_idx,
                  float *topk_w, float *h_amax, void *workspace, size_t workspace_bytes,
                  void *stream);

/* Host-only check of moe_forward's arguments (everything but the workspace size). */
int32_t moe_forward_validate(const moe_forward_args *a);

/* Bytes of device workspace moe_forward needs; depends on the size fields only (fmt, T, D,
 * F, E, top_k, e_begin, e_end) and flags, and is 0 if those are invalid or T = 0. */
size_t moe_forward_workspace_bytes(const moe_forward_args *a);

/* Fills *info for these arguments (the size fields, fmt and flags; pointers unused).
 * Returns MOE_OK or the status moe_forward would return for them. Host only. */
int32_t moe_forward_plan(const moe_forward_args *a, moe_plan_info *info);

/*
 * MoE layer forward over the local experts [e_begin, e_end):
 *  1. slots (t, j) with topk_idx[t][j] local are grouped by expert, stable in t*top_k+j;
 *  2. hidden states are quantised once per token to the layer's format (NVFP4 with
 *     one tensor scale over all of h, MXFP8 and MXFP4 per 32-block, FP8 per token row);
 *     W4A16 and BF16 use the bf16 hidden states as they are;
 *  3. gate_up GEMM per expert (fp32 accumulation; NVFP4 sums are multiplied by
 *     fl32(s_h * s_gate_up[e]), W4A16 sums by s_gate_up[e], FP8 sums by
 *     fl32(s_token * s_channel)), then h = SwiGLU = g * u / (1 + exp(-g));
 *  4. h is quantised to the layer's format (NVFP4: one tensor scale over all S rows;
 *     FP8: one scale per slot row); W4A16 and BF16 round it to bf16 (nearest, ties to
 *     even);
 *  5. down GEMM per expert (NVFP4: times fl32(s_inter * s_down[e]); W4A16: times
 *     s_down[e]; FP8: times fl32(s_row * s_channel)) -> y fp32;
 *  6. out[t] = sum over the token's local slots, j ascending, of topk_w[t][j] * y.
 * Requires D and F multiples of 128 (else MOE_ERR_UNSUPPORTED), and for MXFP4 and FP8
 * also D a multiple of 256 (their GEMMs run on the scaled MFMA in 256-row weight tiles),
 * for MXFP4 also D, F <= 8192 (its kernel holds a tile's E8M0 activation scales for the
 * whole K in LDS; MXFP8 beyond that runs the exact route),
 * 1 <= top_k <= 8, 0 <= e_begin < e_end <= E. gate_up/down must match fmt (NVFP4 for
 * W4A16) and shapes.
 * T = 0 is a no-op.
 */
int32_t moe_forward(const moe_forward_args *a, void *stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same layer and
 * kernels, with the workspace taken from the library's own static device array of
 * MOE_STATIC_SCRATCH_BYTES bytes instead of a->workspace (ignored, may be NULL).
 * It calls no allocating routine. Each GPU the library runs on holds its own copy of
 * the array until the process ends; its address on the current device is looked up on
 * the first call there, so `stream` must belong to the current device.
 * Returns MOE_ERR_WORKSPACE if moe_forward_workspace_bytes(a) exceeds the array (64 MiB
 * covers decode batches of up to about 400 tokens at d_model 4096, d_ff 2560, top-8),
 * otherwise what moe_forward returns. Every call on a GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (different streams, or
 * different host threads) race and must be serialised by the caller.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int32_t moe_forward_static(const moe_forward_args *a, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BLOCK_SCALED_MOE_H */
