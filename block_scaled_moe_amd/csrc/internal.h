// internal.h - launchers shared between the kernel files and the host API.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Device control block at the head of the forward workspace.
struct Ctrl {
    int32_t S;           // local token-slots
    int32_t n_tiles;     // M-tiles of the grouped GEMMs
    uint32_t amax_a;     // max |h| (fp32 bits) when computed by the forward itself
    uint32_t amax_i;     // max |SwiGLU output| over the S rows (fp32 bits), NVFP4
    int32_t pad[60];
};

// Quantisation of the hidden states h [T][D] to the layer's format (act_quant.h): run by
// its own launch or by extra workgroups of the permutation's first launch. kActFP8 is E4M3
// with one fp32 scale per token row, one wave per row; the others one thread per block.
constexpr int32_t kActNone = 0, kActNVFP4 = 1, kActMXFP8 = 2, kActMXFP4 = 3, kActFP8 = 4;
struct ActQuant {
    int32_t fmt;                // kAct*; kActNone: no job
    int32_t T, D;
    const uint16_t *h;          // bf16 [T][D]
    const uint32_t *amax_bits;  // NVFP4: max |h| (fp32 bits)
    uint8_t *codes, *scales;    // [T][D/2] or [T][D]; [T][D/16] or [T][D/32] (FP8: no scales)
    void *deq;                  // NVFP4: exact fp16 values [T][D]; MXFP8: exact bf16 values or NULL
    float *tscale_out;          // NVFP4: [1] the tensor scale
    float *row_scales;          // FP8: [T] the row scales
};
// the job on its own launch
hipError_t launch_act_quant(const ActQuant &q, hipStream_t s);

// ---- weight / activation quantisers (quant.hip)
hipError_t launch_fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s);
hipError_t launch_amax_bf16_rows(const uint16_t *x, int64_t rows, int64_t K, int64_t groups,
                                 uint32_t *amax_bits, hipStream_t s);
hipError_t launch_quant_weights_nvfp4(const uint16_t *w, int32_t E, int32_t N, int32_t K,
                                      const uint32_t *amax_bits, uint8_t *codes, uint8_t *scales,
                                      hipStream_t s);
hipError_t launch_finish_tensor_scale(float *ts_inout, int32_t n, hipStream_t s);
hipError_t launch_quant_weights_mxfp8(const uint16_t *w, int32_t E, int32_t N, int32_t K,
                                      uint8_t *codes, uint8_t *scales, hipStream_t s);
// bf16 weights copied into the packed tile layout (layout.h, 128 bytes per row slot)
hipError_t launch_pack_weights_bf16(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *codes, hipStream_t s);
// row-major pre-quantised codes and scales (fmt 1 NVFP4, 2 MXFP8, 3 MXFP4; 6 FP8: codes
// only, in the MXFP8 order) into the packed tile layout (layout.h); a pure byte reordering
hipError_t launch_pack_rowmajor(int fmt, const uint8_t *src_codes, const uint8_t *src_scales, int32_t E, int32_t N,
                                int32_t K, uint8_t *codes, uint8_t *scales, hipStream_t s);
hipError_t launch_quant_weights_mxfp4(const uint16_t *w, int32_t E, int32_t N, int32_t K,
                                      uint8_t *codes, uint8_t *scales, hipStream_t s);
// FP8 weights: E4M3 codes in the MXFP8 tile layout and one fp32 scale per output channel
// (row), channel_scales [E][N]
hipError_t launch_quant_weights_fp8(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *codes,
                                    float *channel_scales, hipStream_t s);
// FP8 intermediate: rows [0, ctrl->S) of x [*][F] fp32 -> E4M3 codes [S][F] and fp32 row scales [S]
hipError_t launch_quant_inter_fp8(const float *x, int32_t max_rows, int32_t F, const Ctrl *ctrl, uint8_t *codes,
                                  float *row_scales, hipStream_t s);
// intermediate [rows <= ctrl->S][F] fp32 -> NVFP4 (tensor scale from ctrl->amax_i)
hipError_t launch_quant_inter_nvfp4(const float *x, int32_t max_rows, int32_t F, const Ctrl *ctrl,
                                    uint8_t *codes, uint8_t *scales, _Float16 *deq, float *tscale_out,
                                    hipStream_t s);

// ---- router (route.hip)
// Workspace plan of one moe_route call (byte offsets into the caller's workspace).
struct RoutePlan {
    bool screen;          // MFMA screening + exact candidates (large T), else all exact
    int32_t Ep, n_parts;  // padded expert count; 64-wide K blocks of the weight norms
    size_t off_wk8, off_exact, off_logits, off_wpart, off_hn, off_wn, bytes;
};
RoutePlan route_plan(int32_t T, int32_t D, int32_t E);
// logits_out: fp32 [T][E] exact logits, or NULL; amax_bits: max |h| (fp32 bits, the
// route's first kernel zeroes it) or NULL
hipError_t launch_route(const RoutePlan &p, int32_t T, int32_t D, int32_t E, int32_t k, const uint16_t *h,
                        const uint16_t *wr, const float *bias, float *logits_out, int32_t *idx, float *w,
                        uint32_t *amax_bits, void *workspace, hipStream_t s);

// ---- permutation (permute.hip)
struct PermuteArgs {
    int32_t T, k, e_begin, n_loc;
    int32_t chunk_tokens, n_chunks;
    int32_t bm;          // M-tile rows of the grouped GEMMs
    int32_t max_tiles;
    const int32_t *idx;  // [T][k]
    int32_t *chunk_counts;  // [n_chunks][n_loc]
    int32_t *counts;        // [n_loc]
    int32_t *offsets;       // [n_loc + 1]
    int32_t *tile_expert;   // [max_tiles]  local expert of each M-tile
    int32_t *tile_row0;     // [max_tiles]  first sorted position of each M-tile
    int32_t *sorted_slot;   // [T*k]
    int32_t *slot_pos;      // [T*k]  sorted position of each slot or -1
    Ctrl *ctrl;
    ActQuant quant;         // hidden-state quantisation carried by extra workgroups of the
                            // first launch (fmt kActNone: none)
};
hipError_t launch_permute(const PermuteArgs &a, hipStream_t s);
// one-workgroup variant for T*k <= 8192 and <= 1024 local experts; also clears the
// control block's accumulators (no separate fill needed)
bool permute_small_ok(int32_t T, int32_t k, int32_t n_loc);
hipError_t launch_permute_small(const PermuteArgs &a, hipStream_t s);

// ---- grouped GEMMs (gemm.hip)
// Operand formats of the 16-bit-expansion kernels.
//  kFmtNV:  NVFP4 weights and activations (W4A4): fp16 operands, f16 MFMA
//  kFmtMX8: MXFP8 weights and activations: bf16 operands, bf16 MFMA
//  kFmtA16: NVFP4 weights with bf16 activations (W4A16; vLLM recipe
//           "thinkingmachines/Inkling-Small", section "Variants": the weights are
//           dequantised to bf16 on the fly): bf16 operands, bf16 MFMA. A bf16
//           activation is not exact in fp16 in general (range, and 8 significant bits
//           below 2^-14), so the weights are expanded to bf16 instead.
//  kFmtBF:  bf16 weights and activations (the checkpoint's BF16 variant, same section):
//           bf16 operands as stored, no expansion, bf16 MFMA.
constexpr int kFmtNV = 0, kFmtMX8 = 1, kFmtA16 = 2, kFmtBF = 3;

struct GemmArgs {
    const Ctrl *ctrl;
    const int32_t *tile_expert, *tile_row0, *offsets, *sorted_slot;
    int32_t top_k;
    int32_t gather_by_token;  // A row of sorted position p: token sorted_slot[p]/top_k (1) or p (0)
    int32_t N, K;             // weight matrix [N][K] per expert; gate_up: N = 2F
    int32_t e_begin;          // global index of local expert 0
    // A operand: exact 16-bit values of the quantised activations, [rows][K]
    const void *a_vals;       // NVFP4: fp16; MXFP8: bf16; W4A16: the bf16 activations themselves
    // MXFP4 A operand: the codes themselves, [rows][K/2] and E8M0 scales [rows][K/32]
    const uint8_t *a_codes, *a_scales;
    const float *a_tscale;    // NVFP4: [1] activation tensor scale
    const float *a_rscale;    // FP8: fp32 scale of each A row, indexed like the a_codes rows
    // weights (canonical packed layout, global expert index)
    const uint8_t *w_codes, *w_scales;
    const float *w_tscale;    // NVFP4 and W4A16: [E]; FP8: [E][N] channel scales
    // outputs
    float *out_f32;           // gate_up NVFP4 and FP8: SwiGLU [S][F]; down: y [S][N]
    uint32_t *amax_bits;      // gate_up NVFP4: max |SwiGLU|
    uint8_t *o_codes, *o_scales;  // gate_up MXFP8 / MXFP4: quantised SwiGLU [S][F] or [S][F/2], [S][F/32]
    void *o_vals;             // gate_up MXFP8: exact bf16 values of those codes [S][F]; W4A16: bf16 SwiGLU
    float *o_tap;             // gate_up MXFP8 / MXFP4 / W4A16: optional fp32 SwiGLU [S][F]
};
enum class GemmShape { Decode, Prefill };
hipError_t launch_grouped_gemm(const GemmArgs &a, int fm, bool gate_up, GemmShape shape,
                               int32_t max_tiles, hipStream_t s);
int32_t gemm_bm(GemmShape shape);
// prefill-shaped MFMA tiles (gemm_tile.hip): 64- or 128-row M-tiles (by format), 256 or
// 512 weight rows per workgroup
bool tile_gemm_supported(int fm, int32_t K, int32_t N, bool gate_up);
int32_t tile_gemm_bm(int fm);  // rows per M-tile of the tile kernels for operand format fm
hipError_t launch_tile_gemm(const GemmArgs &a, int fm, bool gate_up, int32_t max_tiles, hipStream_t s);
// decode-shaped streaming variant (gemm_stream.hip): 16-row M-tiles, K a multiple of 512
bool stream_gemm_supported(int32_t K, int32_t N, bool gate_up);
hipError_t launch_stream_gemm(const GemmArgs &a, int fm, bool gate_up, int32_t max_tiles, hipStream_t s);

// MXFP4, MXFP8 and FP8 GEMMs on the gfx950 scaled MFMA with the codes (and E8M0 scales)
// as stored (gemm_mx.hip): 128-row M-tiles (mx_gemm_bm), 128 NS weight rows per workgroup
// (mx_gemm_supported checks K % 128, K <= 8192 for the E8M0 formats and the N-block fit);
// A operand: a_codes / a_scales (FP8: a_codes / a_rscale). gate_up writes o_codes /
// o_scales (and o_tap); FP8 writes the SwiGLU output to out_f32 for the row quantiser, its
// sums times fl32(row scale * channel scale).
constexpr int kMxFP4 = 0, kMxFP8 = 1, kMxFP8Rows = 2;
bool mx_gemm_supported(int mode, int32_t K, int32_t N, bool gate_up);
int32_t mx_gemm_bm();
// mode: kMx*; stream_once: decode batches, where each weight panel is read by one M-tile
// (non-temporal weight loads)
hipError_t launch_mx_gemm(const GemmArgs &a, int mode, bool gate_up, bool stream_once, int32_t max_tiles,
                          hipStream_t s);
// The prefill FP8 GEMMs on 256 x 256 workgroup tiles (gemm_fp8_wide.hip): same operands,
// shapes (mx_gemm_supported) and results as launch_mx_gemm's kMxFP8Rows, 256-row M-tiles
// (fp8_wide_gemm_bm).
int32_t fp8_wide_gemm_bm();
hipError_t launch_fp8_wide_gemm(const GemmArgs &a, bool gate_up, int32_t max_tiles, hipStream_t s);
// The prefill bf16-expert GEMMs on 256 x 256 workgroup tiles (gemm_bf16_wide.hip): the
// arithmetic and results of launch_tile_gemm's kFmtBF, 256-row M-tiles (bf16_wide_gemm_bm),
// K % 64 == 0 and 256-row weight blocks (bf16_wide_gemm_supported).
int32_t bf16_wide_gemm_bm();
bool bf16_wide_gemm_supported(int32_t K, int32_t N, bool gate_up);
hipError_t launch_bf16_wide_gemm(const GemmArgs &a, bool gate_up, int32_t max_tiles, hipStream_t s);

// ---- combine (combine.hip)
hipError_t launch_combine(int32_t T, int32_t D, int32_t k, const int32_t *slot_pos, const float *w,
                          const float *y, float *out, hipStream_t s);

}  // namespace moe
