"""Helpers shared by the GPU parity tests: device transfer of the seeded inputs and
the oracle side of each comparison. Inputs come from synth (host), expected values
from oracle/ only."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) or other numpy arrays -> device tensor (same bytes)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def untile(a: np.ndarray) -> np.ndarray:
    """Packed weight bytes [E][N/32][K/64][32][b] (tiled layout of include/moe.h), or
    [E][N/32][K/64][2][32][b] (MXFP4: the two 32-column halves apart) -> the row-major
    [E][N][K/64 * 2b or b] arrays the oracle produces (a pure reordering)."""
    if a.ndim == 6:
        E, nb, kb, h, r, b = a.shape
        return np.ascontiguousarray(a.transpose(0, 1, 4, 2, 3, 5)).reshape(E, nb * r, kb * h * b)
    E, nb, kb, r, b = a.shape
    return np.ascontiguousarray(a.transpose(0, 1, 3, 2, 4)).reshape(E, nb * r, kb * b)


def rms(x: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.asarray(x, np.float64) ** 2)))


def report(name: str, **kv):
    print(name + ": " + ", ".join(f"{k}={v}" for k, v in kv.items()), flush=True)


def case_inputs(wl: synth.Workload):
    """Host inputs of a small workload: hidden, router weight, bias and all expert masters."""
    return (wl.hidden(), wl.router_weight(), wl.router_bias(), wl.gate_up_master(0, wl.E),
            wl.down_master(0, wl.E))


def check_intermediate_codes(fmt: str, inter: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                             tscale: float | None):
    """The GPU's intermediate codes equal the oracle quantiser applied to the GPU's own
    pre-quantisation fp32 values (bit-exact), for the S computed rows."""
    if fmt in ("w4a16", "bf16"):
        # bf16 rounding of the GPU's own fp32 values (no scales)
        oc = oracle.round_bf16(inter)
        bad = int(np.count_nonzero(oc != np.asarray(codes).view(np.uint16)))
        assert bad == 0, f"intermediate bf16 values differ: {bad}"
        return
    if fmt == "fp8":  # scales: the fp32 row scales
        oc, ors = oracle.quant_fp8_rows(inter)
        bad_c = int(np.count_nonzero(oc != codes))
        bad_s = int(np.count_nonzero(ors.view(np.uint32) != np.asarray(scales, np.float32).view(np.uint32)))
        assert bad_c == 0 and bad_s == 0, f"intermediate codes differ: {bad_c} code bytes, {bad_s} row scales"
        return
    if fmt == "nvfp4":
        oc, os_, ots = oracle.quant_nvfp4(inter)
        assert np.float32(tscale) == ots, f"intermediate tensor scale {tscale} != {ots}"
    elif fmt == "mxfp4":
        oc, os_ = oracle.quant_mxfp4(inter)
    else:
        oc, os_ = oracle.quant_mxfp8(inter)
    bad_c = int(np.count_nonzero(oc != codes))
    bad_s = int(np.count_nonzero(os_ != scales))
    assert bad_c == 0 and bad_s == 0, f"intermediate codes differ: {bad_c} code bytes, {bad_s} scale bytes"


def check_outputs(fmt: str, out: np.ndarray, ref: np.ndarray, idx: np.ndarray, w: np.ndarray, gpu_inter_codes,
                  gpu_inter_scales, gpu_inter_tscale, oracle_inter_codes, oracle_inter_scales, sorted_slot,
                  down: dict, *, D: int, F: int, E: int, e_begin: int, e_end: int, rows=None,
                  min_clean_frac: float = 0.5, max_flip_frac: float = 1e-3, max_rel_rms: float = 2e-3):
    """Output parity with intermediate-code flips accounted for.

    The intermediate codes are a rounding of fp32 sums; the GPU sums in a different order
    than the oracle's fp64, so a value on a rounding boundary can land on the neighbouring
    code ("flip"), and one flip moves the affected outputs by up to ~1e-2 x RMS.
     1. stage-wise: the oracle's down projection and combine fed the GPU's intermediate
        codes match the GPU output on every token, to 2e-3 x RMS;
     2. independent: tokens none of whose slots holds a flipped intermediate row match
        the fully independent oracle output, to 2e-3 x RMS;
     3. flips stay rare (< max_flip_frac of the intermediate elements); for the 4- and 8-bit code
        formats at least min_clean_frac of the compared tokens have no flipped row (so
        check 2 covers most of the batch). A bf16 intermediate (W4A16, bf16 experts) flips
        by one bf16 ulp (2^-8 relative) wherever the two sums straddle a rounding
        boundary, which reaches most tokens of a batch, and so do the MXFP8 sums of the
        scaled FP8 MFMA (callers pass min_clean_frac 0): check 4 is the one that bounds
        them;
     4. over all tokens, flipped ones included, the RMS of the difference from the fully
        independent output stays within max_rel_rms x RMS.
    rows: optional token subset to compare (the others are not computed by the oracle).
    FP8: the *_inter_scales are the fp32 row scales [S] (a differing one flips its row).
    Returns (stage error / RMS, independent error / RMS, flips, tokens excluded)."""
    k = idx.shape[1]
    S = len(sorted_slot)
    if fmt == "fp8":
        stage = oracle.down_combine(fmt, idx, w, gpu_inter_codes, None, gpu_inter_scales, down, D=D, F=F, E=E,
                                    e_begin=e_begin, e_end=e_end)
    else:
        stage = oracle.down_combine(fmt, idx, w, gpu_inter_codes, gpu_inter_scales, gpu_inter_tscale, down, D=D, F=F,
                                    E=E, e_begin=e_begin, e_end=e_end)
    sel = np.arange(out.shape[0]) if rows is None else np.asarray(rows)
    r_stage = rms(stage[sel])
    e_stage = float(np.abs(out[sel] - stage[sel]).max()) / r_stage
    assert e_stage <= 2e-3, f"stage-wise output error {e_stage:.2e} x RMS"
    if fmt in ("w4a16", "bf16"):
        gpu_inter_codes = np.asarray(gpu_inter_codes).view(np.uint16)
        oracle_inter_codes = np.asarray(oracle_inter_codes).view(np.uint16)
    cb = gpu_inter_codes.reshape(S, -1) != oracle_inter_codes.reshape(S, -1)
    sb = (np.zeros_like(cb) if gpu_inter_scales is None
          else gpu_inter_scales.reshape(S, -1) != oracle_inter_scales.reshape(S, -1))
    flipped_rows = np.nonzero(cb.any(1) | sb.any(1))[0]
    flips = int(cb.sum())  # differing code bytes (one byte holds two E2M1 codes in the 4-bit formats)
    assert flips <= max_flip_frac * S * F, f"{flips} intermediate code flips in {S * F} elements"
    bad_tokens = set((sorted_slot[flipped_rows] // k).tolist())
    keep = np.array([t for t in sel if t not in bad_tokens], dtype=np.int64)
    if fmt not in ("w4a16", "bf16"):
        assert len(keep) >= min_clean_frac * len(sel), f"{len(sel) - len(keep)} of {len(sel)} tokens reach a flipped row"
    r_ref = rms(ref[sel])
    e_ind = float(np.abs(out[keep] - ref[keep]).max()) / r_ref if len(keep) else 0.0
    assert e_ind <= 2e-3, f"independent output error {e_ind:.2e} x RMS on tokens without flips"
    rel_rms = rms(out[sel] - ref[sel]) / r_ref
    assert rel_rms <= max_rel_rms, f"independent output RMS error {rel_rms:.2e} x RMS"
    return e_stage, e_ind, flips, len(sel) - len(keep)


def device_weights(wl: synth.Workload, device="cuda"):
    """Packed gate_up and down of all experts of a workload, the bf16 masters drawn on the
    GPU (same bytes as the host generator) in chunks of about 1 GiB and quantised there."""
    import block_scaled_moe_amd as moe
    E, D, F = wl.E, wl.D, wl.F
    gu = moe.PackedWeights.empty(wl.fmt, E, 2 * F, D, device=device)
    dn = moe.PackedWeights.empty(wl.fmt, E, D, F, device=device)
    chunk = max(1, min(E, (1 << 30) // (2 * F * D * 2)))
    buf = torch.empty(chunk * 2 * F * D, dtype=torch.int16, device=device)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        n = e1 - e0
        g = buf[: n * 2 * F * D]
        wl.gate_up_master_device(e0, e1, g)
        moe.quantize_weights(wl.fmt, g.view(n, 2 * F, D), out=gu.experts(e0, e1))
        d = buf[: n * D * F]
        wl.down_master_device(e0, e1, d)
        moe.quantize_weights(wl.fmt, d.view(n, D, F), out=dn.experts(e0, e1))
    torch.cuda.synchronize()
    del buf
    return gu, dn


# Bound on the SwiGLU intermediate's difference from the oracle's fp64 sums, relative to
# its largest value: fp32 sums of exact products (every route but one) stay near 1e-7;
# the scaled FP8 MFMA's sums are within about 2e-6 of the sum of |products|
# (tests/test_gpu_fp8_mfma_accuracy.py), which is 1e-5 to 3e-5 of the intermediate's
# maximum at K = 256 to 4096.
INTER_TOL_EXACT = 1e-5
INTER_TOL_SCALED_FP8 = 1e-4
# Bound on intermediate code flips per element. fp32 sums of exact products flip about
# 1e-6 to 1e-5 of the elements (a sum within an ulp of a rounding boundary). The scaled
# FP8 MFMA's error per 64-wide chunk is about 2e-6 of the chunk's sum of |products| and
# averages over chunks only as 1 / sqrt(chunks), so at K = 256 (4 chunks) an element's
# error is about 1e-6 of the sum of |products| and 1e-3 to 1.5e-3 of the elements flip
# (5e-4 at K = 4096).
FLIP_FRAC_EXACT = 1e-3
FLIP_FRAC_SCALED_FP8 = 5e-3
# Bound on the RMS of the output's difference from the fully independent oracle output,
# relative to its RMS. A flip moves one intermediate element by one code step (1/16 to
# 1/8 of its value), so the RMS difference grows as about 0.1 x sqrt(flip fraction):
# 3.4e-3 at the 1.4e-3 flips of K = 256 on the scaled FP8 MFMA; the exact routes stay
# below 2e-4.
REL_RMS_EXACT = 2e-3
REL_RMS_SCALED_FP8 = 1e-2


def scaled_fp8(layer) -> bool:
    """The layer's GEMMs run E4M3 codes (MXFP8 or FP8) on the scaled FP8 MFMA (moe_forward's
    own plan)."""
    return layer.fmt in ("mxfp8", "fp8") and layer.plan()["gate_up_kernel"] in ("mx_gemm_kernel",
                                                                                "fp8_wide_gemm_kernel")


def output_bounds(native8: bool) -> dict:
    """check_outputs bounds for a layer on the scaled FP8 MFMA or on an exact-sum route."""
    if native8:
        return dict(min_clean_frac=0.0, max_flip_frac=FLIP_FRAC_SCALED_FP8, max_rel_rms=REL_RMS_SCALED_FP8)
    return dict(min_clean_frac=0.5, max_flip_frac=FLIP_FRAC_EXACT, max_rel_rms=REL_RMS_EXACT)
