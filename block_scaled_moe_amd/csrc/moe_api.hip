// moe_api.hip - host side of the C ABI declared in include/moe.h: argument
// validation (pure host code, no HIP call), the forward workspace plan, and the
// launch sequence on the caller's stream.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "internal.h"

using namespace moe;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int32_t to_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                                \
    do {                                             \
        const hipError_t err_ = (expr);              \
        if (err_ != hipSuccess) return MOE_ERR_HIP;  \
    } while (0)

// Rows per expert above which the grouped GEMMs use the 128-row tile.
constexpr int32_t kPrefillRowsPerExpert = 48;

// MXFP8 decode batches on the scaled FP8 MFMA kernel (1) or on the streaming kernel with
// the exact bf16 expansion (0)
#ifndef MOE_MX8_DECODE_NATIVE
#define MOE_MX8_DECODE_NATIVE 1
#endif
// FP8 outside decode on the 256 x 256 tiles of gemm_fp8_wide.hip (1) or on the 128-row
// tiles of gemm_mx.hip (0). The same tiles for MXFP8 (weight and activation scales staged
// alongside) measured slower than gemm_mx.hip on the skewed 16K-token layer.
#ifndef MOE_FP8_WIDE
#define MOE_FP8_WIDE 1
#endif
// bf16 experts outside decode on the 256 x 256 tiles of gemm_bf16_wide.hip (1) or on the
// 64-row tiles of gemm_tile.hip (0)
#ifndef MOE_BF16_WIDE
#define MOE_BF16_WIDE 1
#endif

struct Plan {
    GemmShape shape;
    bool scaled;  // MXFP4 / MXFP8 / FP8 on the scaled MFMA with the codes as stored (gemm_mx.hip)
    bool wide;    // FP8 outside decode: the 256 x 256 tiles (gemm_fp8_wide.hip)
    bool bfwide;  // bf16 experts outside decode: the 256 x 256 tiles (gemm_bf16_wide.hip)
    bool tiled;   // prefill on the MFMA tile kernels (64- or 128-row M-tiles), or scaled
    int32_t n_loc, chunk_tokens, n_chunks, bm, max_tiles;
    size_t ctrl, chunk_counts, counts, offsets, tile_expert, tile_row0, sorted_slot, slot_pos;
    size_t a_codes, a_scales, a_tscale, a16;
    size_t inter32, i_codes, i_scales, i_tscale, i16, y;
    size_t total;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// operand format of the 16-bit-expansion GEMM kernels for a layer format (not MXFP4)
int gemm_fm(int32_t fmt) {
    return fmt == MOE_FMT_NVFP4 ? kFmtNV : fmt == MOE_FMT_W4A16 ? kFmtA16 : fmt == MOE_FMT_BF16 ? kFmtBF : kFmtMX8;
}

Plan make_plan(const moe_forward_args *a) {
    Plan p{};
    const int64_t T = a->T, D = a->D, F = a->F, k = a->top_k, TK = T * k;
    const bool nv = a->fmt == MOE_FMT_NVFP4, mx4 = a->fmt == MOE_FMT_MXFP4, f8 = a->fmt == MOE_FMT_FP8;
    const bool a16 = a->fmt == MOE_FMT_W4A16 || a->fmt == MOE_FMT_BF16;  // bf16 activations
    const bool byte_codes = a->fmt == MOE_FMT_MXFP8 || f8;               // one code byte per value
    p.n_loc = a->e_end - a->e_begin;
    p.shape = (TK / a->E >= kPrefillRowsPerExpert) ? GemmShape::Prefill : GemmShape::Decode;
    // MXFP4 and FP8 always run the scaled MFMA kernels (validate_shape checks the fit);
    // MXFP8 the scaled-FP8 ones unless the caller asks for exact sums or the shape does not
    // fit them
    const int mx_mode = mx4 ? kMxFP4 : (f8 ? kMxFP8Rows : kMxFP8);
    const bool mx_fit = mx_gemm_supported(mx_mode, a->D, 2 * a->F, true) && mx_gemm_supported(mx_mode, a->F, a->D, false);
    p.scaled = mx4 || f8 ||
               (a->fmt == MOE_FMT_MXFP8 && !(a->flags & MOE_FLAG_EXACT_SUMS) && mx_fit &&
                (p.shape == GemmShape::Prefill || MOE_MX8_DECODE_NATIVE));
    p.tiled = p.scaled || (p.shape == GemmShape::Prefill && tile_gemm_supported(gemm_fm(a->fmt), a->D, 2 * a->F, true) &&
                           tile_gemm_supported(gemm_fm(a->fmt), a->F, a->D, false));
    p.wide = f8 && p.shape == GemmShape::Prefill && MOE_FP8_WIDE;
    p.bfwide = a->fmt == MOE_FMT_BF16 && p.shape == GemmShape::Prefill && MOE_BF16_WIDE &&
               bf16_wide_gemm_supported(a->D, 2 * a->F, true) && bf16_wide_gemm_supported(a->F, a->D, false);
    p.bm = p.wide ? fp8_wide_gemm_bm() : p.bfwide ? bf16_wide_gemm_bm() : p.scaled ? mx_gemm_bm() : (p.tiled ? tile_gemm_bm(gemm_fm(a->fmt)) : gemm_bm(p.shape));
    int32_t ct = (int32_t)(T / 256);
    p.chunk_tokens = ct < 8 ? 8 : (ct > 64 ? 64 : ct);
    p.n_chunks = (int32_t)((T + p.chunk_tokens - 1) / p.chunk_tokens);
    p.max_tiles = (int32_t)(p.n_loc + TK / p.bm + 1);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += up256(bytes);
        return at;
    };
    p.ctrl = take(sizeof(Ctrl));
    p.chunk_counts = take(sizeof(int32_t) * (size_t)p.n_chunks * p.n_loc);
    p.counts = take(sizeof(int32_t) * p.n_loc);
    p.offsets = take(sizeof(int32_t) * (p.n_loc + 1));
    p.tile_expert = take(sizeof(int32_t) * p.max_tiles);
    p.tile_row0 = take(sizeof(int32_t) * p.max_tiles);
    p.sorted_slot = take(sizeof(int32_t) * TK);
    p.slot_pos = take(sizeof(int32_t) * TK);
    // W4A16 and bf16 experts keep the hidden states as they are and the intermediate in
    // bf16 (i16 only); FP8's scales are one fp32 per row
    p.a_codes = a16 ? 0 : take(byte_codes ? T * D : T * D / 2);
    p.a_scales = a16 ? 0 : take(f8 ? sizeof(float) * T : (nv ? T * D / 16 : T * D / 32));
    p.a_tscale = take(sizeof(float));
    p.a16 = (p.scaled || a16) ? 0 : take(2 * T * D);  // exact 16-bit values of the hidden-state codes
    p.inter32 = (nv || f8) ? take(sizeof(float) * TK * F) : 0;
    p.i_codes = a16 ? 0 : take(byte_codes ? TK * F : TK * F / 2);
    p.i_scales = a16 ? 0 : take(f8 ? sizeof(float) * TK : (nv ? TK * F / 16 : TK * F / 32));
    p.i_tscale = take(sizeof(float));
    p.i16 = p.scaled ? 0 : take(2 * TK * F);  // exact 16-bit values of the intermediate (codes)
    p.y = take(sizeof(float) * TK * D);
    p.total = off;
    return p;
}

// The kernel family each GEMM of a plan runs (what run_gemm launches).
enum class Kernel { Wide, BfWide, Scaled, Tile, Stream, Grouped };

Kernel gemm_kernel(const Plan &P, int32_t K, int32_t N, bool gate_up) {
    if (P.wide) return Kernel::Wide;
    if (P.bfwide) return Kernel::BfWide;
    if (P.scaled) return Kernel::Scaled;
    if (P.tiled) return Kernel::Tile;
    if (P.shape == GemmShape::Decode && stream_gemm_supported(K, N, gate_up)) return Kernel::Stream;
    return Kernel::Grouped;
}

const char *kernel_name(Kernel k) {
    switch (k) {
        case Kernel::Wide: return "fp8_wide_gemm_kernel";
        case Kernel::BfWide: return "bf16_wide_gemm_kernel";
        case Kernel::Scaled: return "mx_gemm_kernel";
        case Kernel::Tile: return "tile_gemm_kernel";
        case Kernel::Stream: return "stream_gemm_kernel";
        default: return "grouped_gemm_kernel";
    }
}

hipError_t run_gemm(const GemmArgs &g, int32_t fmt, bool gate_up, const Plan &P, hipStream_t s) {
    const int fm = gemm_fm(fmt);
    switch (gemm_kernel(P, g.K, g.N, gate_up)) {
        case Kernel::Wide: return launch_fp8_wide_gemm(g, gate_up, P.max_tiles, s);
        case Kernel::BfWide: return launch_bf16_wide_gemm(g, gate_up, P.max_tiles, s);
        case Kernel::Scaled:
            return launch_mx_gemm(g, fmt == MOE_FMT_MXFP8 ? kMxFP8 : (fmt == MOE_FMT_FP8 ? kMxFP8Rows : kMxFP4), gate_up,
                                  P.shape == GemmShape::Decode, P.max_tiles, s);
        case Kernel::Tile: return launch_tile_gemm(g, fm, gate_up, P.max_tiles, s);
        case Kernel::Stream: return launch_stream_gemm(g, fm, gate_up, P.max_tiles, s);
        default: return launch_grouped_gemm(g, fm, gate_up, P.shape, P.max_tiles, s);
    }
}

int32_t check_packed(const moe_packed &w, int32_t fmt, int32_t E, int32_t N, int32_t K) {
    if (w.fmt != fmt || w.E != E || w.N != N || w.K != K) return MOE_ERR_INVALID_ARG;
    const bool need_scales = fmt != MOE_FMT_BF16 && fmt != MOE_FMT_FP8;  // bf16 and FP8 have no block scales
    const bool need_tscale = fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_FP8;
    if (!w.codes || (need_scales && !w.scales) || (need_tscale && !w.tensor_scale)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(w.codes) || (w.scales && !aligned16(w.scales)) ||
        (w.tensor_scale && ((uintptr_t)w.tensor_scale & 3u)))
        return MOE_ERR_ALIGNMENT;
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int32_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int32_t moe_quantize_weights(const uint16_t *w, moe_packed *out, void *stream) {
    if (!out || !w) return MOE_ERR_INVALID_ARG;
    const int32_t fmt = out->fmt, E = out->E, N = out->N, K = out->K;
    if (fmt != MOE_FMT_NVFP4 && fmt != MOE_FMT_MXFP8 && fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_BF16 &&
        fmt != MOE_FMT_FP8)
        return MOE_ERR_INVALID_ARG;
    if (E <= 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
    if (N % 32 || K % 64) return MOE_ERR_INVALID_ARG;  // tiled layout of include/moe.h
    const bool need_scales = fmt != MOE_FMT_BF16 && fmt != MOE_FMT_FP8;
    if (!out->codes || (need_scales && !out->scales) ||
        ((fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_FP8) && !out->tensor_scale))
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(out->codes) || ((uintptr_t)out->tensor_scale & 3u)) return MOE_ERR_ALIGNMENT;
    hipStream_t s = (hipStream_t)stream;
    if (fmt == MOE_FMT_BF16) return to_status(launch_pack_weights_bf16(w, E, N, K, out->codes, s));
    if (fmt == MOE_FMT_FP8) return to_status(launch_quant_weights_fp8(w, E, N, K, out->codes, out->tensor_scale, s));
    if (fmt == MOE_FMT_MXFP8)
        return to_status(launch_quant_weights_mxfp8(w, E, N, K, out->codes, out->scales, s));
    if (fmt == MOE_FMT_MXFP4)
        return to_status(launch_quant_weights_mxfp4(w, E, N, K, out->codes, out->scales, s));
    uint32_t *amax = reinterpret_cast<uint32_t *>(out->tensor_scale);  // amax bits, then the scale
    MOE_TRY(launch_fill_u32(amax, 0u, E, s));
    MOE_TRY(launch_amax_bf16_rows(w, (int64_t)E * N, K, E, amax, s));
    MOE_TRY(launch_quant_weights_nvfp4(w, E, N, K, amax, out->codes, out->scales, s));
    return to_status(launch_finish_tensor_scale(out->tensor_scale, E, s));
}

int32_t moe_pack_weights(const moe_rowmajor *in, moe_packed *out, void *stream) {
    if (!in || !out) return MOE_ERR_INVALID_ARG;
    const int32_t fmt = in->fmt, E = in->E, N = in->N, K = in->K;
    if (fmt != MOE_FMT_NVFP4 && fmt != MOE_FMT_MXFP8 && fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_BF16 &&
        fmt != MOE_FMT_FP8)
        return MOE_ERR_INVALID_ARG;
    if (out->fmt != fmt || out->E != E || out->N != N || out->K != K) return MOE_ERR_INVALID_ARG;
    if (E <= 0 || N <= 0 || K <= 0 || N % 32 || K % 64) return MOE_ERR_INVALID_ARG;
    const bool scaled = fmt != MOE_FMT_BF16 && fmt != MOE_FMT_FP8;  // block scales to move
    const bool ts = fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_FP8;      // tensor / channel scales to copy
    if (!in->codes || !out->codes || (scaled && (!in->scales || !out->scales)) ||
        (ts && (!in->tensor_scale || !out->tensor_scale)))
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(in->codes) || !aligned16(out->codes) || (scaled && !aligned16(out->scales)) ||
        (ts && (((uintptr_t)in->tensor_scale | (uintptr_t)out->tensor_scale) & 3u)))
        return MOE_ERR_ALIGNMENT;
    hipStream_t s = (hipStream_t)stream;
    if (fmt == MOE_FMT_BF16)
        return to_status(launch_pack_weights_bf16(reinterpret_cast<const uint16_t *>(in->codes), E, N, K, out->codes, s));
    MOE_TRY(launch_pack_rowmajor(fmt, in->codes, scaled ? in->scales : nullptr, E, N, K, out->codes,
                                 scaled ? out->scales : nullptr, s));
    if (ts) {
        const size_t n = fmt == MOE_FMT_FP8 ? (size_t)E * N : (size_t)E;  // FP8: one per channel
        MOE_TRY(hipMemcpyAsync(out->tensor_scale, in->tensor_scale, sizeof(float) * n, hipMemcpyDeviceToDevice, s));
    }
    return MOE_OK;
}

size_t moe_route_workspace_bytes(int32_t T, int32_t D, int32_t E) {
    if (T <= 0 || D <= 0 || D % 64 || E <= 0 || E > 1024) return 0;
    return route_plan(T, D, E).bytes;
}

int32_t moe_route(int32_t T, int32_t D, int32_t E, int32_t top_k, const uint16_t *h, const uint16_t *wr,
                  const float *bias, float *logits, int32_t *topk_idx, float *topk_w, float *h_amax,
                  void *workspace, size_t workspace_bytes, void *stream) {
    if (T < 0 || D <= 0 || E <= 0 || E > 1024 || top_k < 1 || top_k > 8 || top_k > E) return MOE_ERR_INVALID_ARG;
    if (D % 64) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!h || !wr || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned16(h) || !aligned16(wr) || !aligned16(topk_idx) || !aligned16(topk_w) ||
        (logits && !aligned16(logits)) || (bias && !aligned16(bias)) || (h_amax && !aligned16(h_amax)))
        return MOE_ERR_ALIGNMENT;
    const RoutePlan plan = route_plan(T, D, E);
    if (!workspace || workspace_bytes < plan.bytes) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGNMENT;
    hipStream_t s = (hipStream_t)stream;
    uint32_t *amax = reinterpret_cast<uint32_t *>(h_amax);  // zeroed by the route's first kernel
    return to_status(launch_route(plan, T, D, E, top_k, h, wr, bias, logits, topk_idx, topk_w, amax, workspace, s));
}

}  // extern "C"

namespace {

// The size fields alone (what the workspace plan depends on).
int32_t validate_shape(const moe_forward_args *a) {
    if (!a) return MOE_ERR_INVALID_ARG;
    if (a->fmt != MOE_FMT_NVFP4 && a->fmt != MOE_FMT_MXFP8 && a->fmt != MOE_FMT_MXFP4 && a->fmt != MOE_FMT_W4A16 &&
        a->fmt != MOE_FMT_BF16 && a->fmt != MOE_FMT_FP8)
        return MOE_ERR_INVALID_ARG;
    if (a->T < 0 || a->D <= 0 || a->F <= 0 || a->E <= 0 || a->E > 4096) return MOE_ERR_INVALID_ARG;
    if (a->top_k < 1 || a->top_k > 8 || a->top_k > a->E) return MOE_ERR_INVALID_ARG;
    if (a->e_begin < 0 || a->e_end <= a->e_begin || a->e_end > a->E) return MOE_ERR_INVALID_ARG;
    if ((int64_t)a->T * a->top_k > INT32_MAX / 2) return MOE_ERR_INVALID_ARG;
    if (a->D % 128 || a->F % 128) return MOE_ERR_UNSUPPORTED;
    if (a->flags & ~(uint32_t)MOE_FLAG_EXACT_SUMS) return MOE_ERR_INVALID_ARG;
    if (a->fmt == MOE_FMT_MXFP4 &&
        !(mx_gemm_supported(kMxFP4, a->D, 2 * a->F, true) && mx_gemm_supported(kMxFP4, a->F, a->D, false)))
        return MOE_ERR_UNSUPPORTED;
    // FP8 runs on the scaled FP8 MFMA only (no exact-sum route)
    if (a->fmt == MOE_FMT_FP8 &&
        ((a->flags & MOE_FLAG_EXACT_SUMS) ||
         !(mx_gemm_supported(kMxFP8Rows, a->D, 2 * a->F, true) && mx_gemm_supported(kMxFP8Rows, a->F, a->D, false))))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_forward_validate(const moe_forward_args *a) {
    const int32_t shape = validate_shape(a);
    if (shape != MOE_OK) return shape;
    if (a->T == 0) return MOE_OK;
    if (!a->h || !a->topk_idx || !a->topk_w || !a->out) return MOE_ERR_INVALID_ARG;
    const int32_t wfmt = a->fmt == MOE_FMT_W4A16 ? MOE_FMT_NVFP4 : a->fmt;  // packed weights' format
    int32_t rc = check_packed(a->gate_up, wfmt, a->E, 2 * a->F, a->D);
    if (rc != MOE_OK) return rc;
    rc = check_packed(a->down, wfmt, a->E, a->D, a->F);
    if (rc != MOE_OK) return rc;
    if (!aligned16(a->h) || !aligned16(a->topk_idx) || !aligned16(a->topk_w) || !aligned16(a->out) ||
        (a->h_amax && !aligned16(a->h_amax)))
        return MOE_ERR_ALIGNMENT;
    if (a->taps && a->taps->inter && !aligned16(a->taps->inter)) return MOE_ERR_ALIGNMENT;
    return MOE_OK;
}

size_t moe_forward_workspace_bytes(const moe_forward_args *a) {
    if (validate_shape(a) != MOE_OK) return 0;
    if (a->T == 0) return 0;
    return make_plan(a).total;
}

int32_t moe_forward_plan(const moe_forward_args *a, moe_plan_info *info) {
    if (!info) return MOE_ERR_INVALID_ARG;
    const int32_t rc = validate_shape(a);
    if (rc != MOE_OK) return rc;
    memset(info, 0, sizeof(*info));
    if (a->T == 0) {
        info->gate_up_kernel = info->down_kernel = "none";
        return MOE_OK;
    }
    const Plan P = make_plan(a);
    info->gate_up_kernel = kernel_name(gemm_kernel(P, a->D, 2 * a->F, true));
    info->down_kernel = kernel_name(gemm_kernel(P, a->F, a->D, false));
    info->m_tile_rows = P.bm;
    info->workspace_bytes = P.total;
    return MOE_OK;
}

}  // extern "C"

namespace {

// The launch sequence of one forward call on the validated arguments `a` with the plan P
// and P.total bytes of device workspace at ws (256-byte aligned).
int32_t run_forward(const moe_forward_args *a, const Plan &P, uint8_t *ws, hipStream_t s) {
    const bool nv = a->fmt == MOE_FMT_NVFP4, mx4 = a->fmt == MOE_FMT_MXFP4, f8 = a->fmt == MOE_FMT_FP8;
    const bool a16 = a->fmt == MOE_FMT_W4A16 || a->fmt == MOE_FMT_BF16;  // bf16 activations
    const int32_t T = a->T, D = a->D, F = a->F, k = a->top_k, TK = T * k;
    Ctrl *ctrl = reinterpret_cast<Ctrl *>(ws + P.ctrl);
    auto I32 = [&](size_t off) { return reinterpret_cast<int32_t *>(ws + off); };
    auto U8 = [&](size_t off) { return ws + off; };
    auto F32 = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
    auto F16 = [&](size_t off) { return reinterpret_cast<_Float16 *>(ws + off); };

    auto mark = [&](int i) -> hipError_t {
        return a->events ? hipEventRecord((hipEvent_t)a->events[i], s) : hipSuccess;
    };
    MOE_TRY(mark(MOE_EV_BEGIN));
    const bool small = permute_small_ok(T, k, P.n_loc);

    // 1. stable grouping of the local slots and the GEMM tile list
    PermuteArgs pa{};
    pa.T = T;
    pa.k = k;
    pa.e_begin = a->e_begin;
    pa.n_loc = P.n_loc;
    pa.chunk_tokens = P.chunk_tokens;
    pa.n_chunks = P.n_chunks;
    pa.bm = P.bm;
    pa.max_tiles = P.max_tiles;
    pa.idx = a->topk_idx;
    pa.chunk_counts = I32(P.chunk_counts);
    pa.counts = I32(P.counts);
    pa.offsets = I32(P.offsets);
    pa.tile_expert = I32(P.tile_expert);
    pa.tile_row0 = I32(P.tile_row0);
    pa.sorted_slot = I32(P.sorted_slot);
    pa.slot_pos = I32(P.slot_pos);
    pa.ctrl = ctrl;

    // 2. hidden states quantised once per token (W4A16 and bf16 experts read them as they
    // are): NVFP4 with one tensor scale over all of h from the router's max |h|; MXFP8
    // also writes its exact bf16 values for the exact route; FP8 one scale per token row.
    // The job rides in extra workgroups of the permutation's first launch; without the
    // router's max |h| an NVFP4 layer takes an amax pass after the permutation and
    // quantises on its own.
    ActQuant q{};
    q.fmt = nv ? kActNVFP4 : (mx4 ? kActMXFP4 : (a16 ? kActNone : (f8 ? kActFP8 : kActMXFP8)));
    q.T = T;
    q.D = D;
    q.h = a->h;
    q.amax_bits = nv ? (a->h_amax ? reinterpret_cast<const uint32_t *>(a->h_amax) : &ctrl->amax_a) : nullptr;
    q.codes = a16 ? nullptr : U8(P.a_codes);
    q.scales = (a16 || f8) ? nullptr : U8(P.a_scales);
    q.row_scales = f8 ? F32(P.a_scales) : nullptr;
    q.deq = nv ? static_cast<void *>(F16(P.a16)) : ((mx4 || a16 || P.scaled) ? nullptr : static_cast<void *>(ws + P.a16));
    q.tscale_out = nv ? F32(P.a_tscale) : nullptr;
    const bool carried = !(nv && !a->h_amax);
    if (carried) pa.quant = q;
    MOE_TRY(small ? launch_permute_small(pa, s) : launch_permute(pa, s));
    if (!carried) {
        MOE_TRY(launch_amax_bf16_rows(a->h, T, D, 1, &ctrl->amax_a, s));  // amax_a cleared by the permutation
        MOE_TRY(launch_act_quant(q, s));
    }

    // 3. gate_up GEMM + SwiGLU (+ MXFP8 intermediate quantisation)
    GemmArgs g{};
    g.ctrl = ctrl;
    g.tile_expert = I32(P.tile_expert);
    g.tile_row0 = I32(P.tile_row0);
    g.offsets = I32(P.offsets);
    g.sorted_slot = I32(P.sorted_slot);
    g.top_k = k;
    g.gather_by_token = 1;
    g.N = 2 * F;
    g.K = D;
    g.e_begin = a->e_begin;
    g.w_codes = a->gate_up.codes;
    g.w_scales = a->gate_up.scales;
    g.w_tscale = a->gate_up.tensor_scale;
    g.a_vals = P.scaled ? nullptr : (a16 ? static_cast<const void *>(a->h) : ws + P.a16);
    g.a_codes = a16 ? nullptr : U8(P.a_codes);
    g.a_scales = (a16 || f8) ? nullptr : U8(P.a_scales);
    g.a_rscale = f8 ? F32(P.a_scales) : nullptr;
    if (f8) {
        g.out_f32 = F32(P.inter32);
        MOE_TRY(mark(MOE_EV_GATE_UP));
        MOE_TRY(run_gemm(g, a->fmt, true, P, s));
        MOE_TRY(mark(MOE_EV_GATE_UP_END));
        // 4. FP8 intermediate: one scale per slot row
        MOE_TRY(launch_quant_inter_fp8(F32(P.inter32), TK, F, ctrl, U8(P.i_codes), F32(P.i_scales), s));
    } else if (nv) {
        g.a_tscale = F32(P.a_tscale);
        g.out_f32 = F32(P.inter32);
        g.amax_bits = &ctrl->amax_i;
        MOE_TRY(mark(MOE_EV_GATE_UP));
        MOE_TRY(run_gemm(g, a->fmt, true, P, s));
        MOE_TRY(mark(MOE_EV_GATE_UP_END));
        // 4. NVFP4 intermediate: one tensor scale over all S rows
        MOE_TRY(launch_quant_inter_nvfp4(F32(P.inter32), TK, F, ctrl, U8(P.i_codes), U8(P.i_scales), F16(P.i16),
                                         F32(P.i_tscale), s));
    } else {
        g.o_codes = a16 ? nullptr : U8(P.i_codes);
        g.o_vals = P.scaled ? nullptr : ws + P.i16;
        g.o_scales = a16 ? nullptr : U8(P.i_scales);
        g.o_tap = a->taps ? a->taps->inter : nullptr;
        MOE_TRY(mark(MOE_EV_GATE_UP));
        MOE_TRY(run_gemm(g, a->fmt, true, P, s));
        MOE_TRY(mark(MOE_EV_GATE_UP_END));
    }

    // 5. down GEMM -> y [S][D]
    GemmArgs d = g;
    d.gather_by_token = 0;
    d.N = D;
    d.K = F;
    d.w_codes = a->down.codes;
    d.w_scales = a->down.scales;
    d.w_tscale = a->down.tensor_scale;
    d.out_f32 = F32(P.y);
    d.amax_bits = nullptr;
    d.o_codes = nullptr;
    d.o_scales = nullptr;
    d.o_tap = nullptr;
    d.o_vals = nullptr;
    d.a_vals = P.scaled ? nullptr : ws + P.i16;
    d.a_codes = a16 ? nullptr : U8(P.i_codes);
    d.a_scales = (a16 || f8) ? nullptr : U8(P.i_scales);
    d.a_rscale = f8 ? F32(P.i_scales) : nullptr;
    d.a_tscale = nv ? F32(P.i_tscale) : nullptr;
    MOE_TRY(mark(MOE_EV_DOWN));
    MOE_TRY(run_gemm(d, a->fmt, false, P, s));
    MOE_TRY(mark(MOE_EV_DOWN_END));

    // 6. weighted combine
    MOE_TRY(launch_combine(T, D, k, I32(P.slot_pos), a->topk_w, F32(P.y), a->out, s));
    MOE_TRY(mark(MOE_EV_END));

    // debug taps
    if (a->taps) {
        const moe_taps *t = a->taps;
        auto cp = [&](void *dst, const void *src, size_t n) -> hipError_t {
            return dst ? hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, s) : hipSuccess;
        };
        MOE_TRY(cp(t->counts, ws + P.counts, sizeof(int32_t) * P.n_loc));
        MOE_TRY(cp(t->offsets, ws + P.offsets, sizeof(int32_t) * (P.n_loc + 1)));
        MOE_TRY(cp(t->sorted_slot, ws + P.sorted_slot, sizeof(int32_t) * (size_t)TK));
        const bool b8 = a->fmt == MOE_FMT_MXFP8 || f8;  // one code byte per value
        if (!a16) MOE_TRY(cp(t->a_codes, ws + P.a_codes, b8 ? (size_t)T * D : (size_t)T * D / 2));
        if (!a16 && !f8) MOE_TRY(cp(t->a_scales, ws + P.a_scales, nv ? (size_t)T * D / 16 : (size_t)T * D / 32));
        if (nv) {
            MOE_TRY(cp(t->a_tscale, ws + P.a_tscale, sizeof(float)));
            MOE_TRY(cp(t->inter_tscale, ws + P.i_tscale, sizeof(float)));
        }
        if (f8) {  // the row scales
            MOE_TRY(cp(t->a_tscale, ws + P.a_scales, sizeof(float) * (size_t)T));
            MOE_TRY(cp(t->inter_tscale, ws + P.i_scales, sizeof(float) * (size_t)TK));
        }
        if (nv || f8) MOE_TRY(cp(t->inter, ws + P.inter32, sizeof(float) * (size_t)TK * F));
        if (a16) {
            MOE_TRY(cp(t->inter_codes, ws + P.i16, 2 * (size_t)TK * F));  // bf16 bit patterns
        } else {
            MOE_TRY(cp(t->inter_codes, ws + P.i_codes, b8 ? (size_t)TK * F : (size_t)TK * F / 2));
            if (!f8) MOE_TRY(cp(t->inter_scales, ws + P.i_scales, nv ? (size_t)TK * F / 16 : (size_t)TK * F / 32));
        }
        MOE_TRY(cp(t->y, ws + P.y, sizeof(float) * (size_t)TK * D));
    }
    return MOE_OK;
}

// Device scratch of moe_forward_static: a file-scope array, so that the call allocates
// nothing. Each GPU the library runs on holds its own copy for the life of the process;
// host code addresses it only through the per-device pointer from hipGetSymbolAddress.
constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on that device.
int32_t static_scratch(uint8_t **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<uint8_t *>(g_scratch_ptr[dev]);
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_forward(const moe_forward_args *a, void *stream) {
    int32_t rc = moe_forward_validate(a);
    if (rc != MOE_OK) return rc;
    if (a->T == 0) return MOE_OK;
    const Plan P = make_plan(a);
    if (!a->workspace || a->workspace_bytes < P.total) return MOE_ERR_WORKSPACE;
    if (((uintptr_t)a->workspace & 255u) != 0) return MOE_ERR_ALIGNMENT;
    return run_forward(a, P, static_cast<uint8_t *>(a->workspace), (hipStream_t)stream);
}

int32_t moe_forward_static(const moe_forward_args *a, void *stream) {
    int32_t rc = moe_forward_validate(a);
    if (rc != MOE_OK) return rc;
    if (a->T == 0) return MOE_OK;
    const Plan P = make_plan(a);
    if (P.total > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
    uint8_t *ws = nullptr;
    rc = static_scratch(&ws);
    if (rc != MOE_OK) return rc;
    return run_forward(a, P, ws, (hipStream_t)stream);
}

}  // extern "C"
