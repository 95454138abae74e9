"""GPU parity at the full sizes of the twelve benchmarked workloads, through the same calls
and launch configuration that bench.py times (moe.route + moe.Layer.forward).

Bit-exact, whole batch: top-k indices of every token, max |h|, the permutation, every
hidden-state code and scale, every intermediate code and scale given the GPU's own fp32
intermediate, and the packed weight bytes of every expert the batch touches.

Expert arithmetic, every slot of every touched local expert, one expert at a time with
fp64 BLAS on the oracle's dequantised operands (its quantised weights, the verified
hidden-state codes):
 - the fp32 SwiGLU intermediate within 1e-5 of the expert's largest value (1e-4 on the
   scaled FP8 MFMA);
 - the per-slot down projection y stage-wise (from the GPU's intermediate codes) within
   2e-3 x the RMS of the expert's y;
 - the layer output stage-wise (that down projection combined in fp64) within 2e-3 x RMS
   on every token;
 - the layer output fully independently: the reference intermediate quantised by the
   oracle over all S rows, projected down and combined in fp64. Intermediate elements
   whose codes differ from the GPU's ("flips": the GPU's fp32 sums and the oracle's fp64
   sums round to neighbouring codes) are counted and reported with the error of the
   tokens they reach; tokens without a flipped row must match within 2e-3 x RMS, and the
   relative RMS error over all tokens must stay within 2e-3 (1e-2 for MXFP8 on the
   scaled FP8 MFMA, whose sums flip about 100 times as many codes; tests/gpu_util.py).
The decode NVFP4, MXFP8 and FP8 workloads are also run through the oracle's own forward
(its routing, permutation, quantisers and fp64 experts) on the experts the batch touches,
and compared with the GPU output stage-wise and independently. FP8's scales are fp32 per
row (tokens, slots) and per weight channel: its "scales" below are those row scales, and
its sums are multiplied by fl32(row scale * channel scale).
"""
import time

import numpy as np
import pytest
import torch

import block_scaled_moe_amd as moe
import oracle
import synth
from gpu_util import (INTER_TOL_EXACT, INTER_TOL_SCALED_FP8, check_intermediate_codes, check_outputs, device_weights,
                      host, output_bounds, report, rms, scaled_fp8, to_dev, untile)

pytestmark = pytest.mark.gpu


def _dequant(fmt, codes, scales):
    """fp64 values of packed codes (NVFP4 without its tensor scale, FP8 without its row or
    channel scales)."""
    if fmt == "fp8":
        return oracle.dequant_fp8_rows(codes)
    if fmt in ("nvfp4", "w4a16"):
        return oracle.dequant_nvfp4(codes, scales, 1.0, with_tensor=False)
    if fmt == "mxfp4":
        return oracle.dequant_mxfp4(codes, scales)
    return oracle.dequant_mxfp8(codes, scales)


def _oracle_expert(wl, e):
    """The oracle's packed weights of expert e (bf16 experts: the masters) as
    (gate_up, down) dicts of [1, N, K] arrays."""
    gm, dm = wl.gate_up_master(e), wl.down_master(e)
    if wl.fmt == "bf16":
        return {"codes": gm, "scales": None, "tensor_scale": None}, {"codes": dm, "scales": None, "tensor_scale": None}
    return oracle.quantize_weights(wl.fmt, gm), oracle.quantize_weights(wl.fmt, dm)


def _values(fmt, w):
    """fp64 [N, K] values of one expert's packed matrix (without the NVFP4 tensor scale or
    the FP8 channel scales)."""
    if fmt == "bf16":
        return synth.bf16_to_f32(w["codes"][0]).astype(np.float64)
    return _dequant(fmt, w["codes"][0], None if w["scales"] is None else w["scales"][0])


def _scale_sums(fmt, sums, w, row_scales, tscale):
    """fp32 sums [rows, N] of one expert times the format's scales, rounded to fp32:
    NVFP4 fl32(tensor scale of the operand * the weights'), W4A16 the weights' tensor scale,
    FP8 fl32(row scale * channel scale); the others none."""
    sums = sums.astype(np.float32)
    if fmt == "nvfp4":
        return (sums * np.float32(np.float32(tscale) * w["tensor_scale"][0])).astype(np.float32)
    if fmt == "w4a16":
        return (sums * np.float32(w["tensor_scale"][0])).astype(np.float32)
    if fmt == "fp8":
        f = (np.asarray(row_scales, np.float32)[:, None] * w["tensor_scale"][0][None, :]).astype(np.float32)
        return (sums * f).astype(np.float32)
    return sums


def _inter_values(fmt, codes, scales):
    """fp64 values of intermediate codes (16-bit formats: bf16 bit patterns)."""
    if fmt in ("w4a16", "bf16"):
        return synth.bf16_to_f32(np.asarray(codes).view(np.uint16)).astype(np.float64)
    return _dequant(fmt, codes, scales)


def _code_flips(fmt, got, ref):
    """(rows with a differing element, number of differing elements) of two intermediate
    code arrays [S][...] (the 4-bit formats hold two elements per byte)."""
    if fmt in ("w4a16", "bf16"):
        d = np.asarray(got).view(np.uint16) != np.asarray(ref).view(np.uint16)
        return d.any(1), int(d.sum())
    if fmt in ("nvfp4", "mxfp4"):
        lo, hi = (got & 0xF) != (ref & 0xF), (got >> 4) != (ref >> 4)
        return (lo | hi).any(1), int(lo.sum()) + int(hi.sum())
    d = got != ref
    return d.any(1), int(d.sum())


def _combine(T, D, k, ss, w, y):
    """out[t] = sum_j w[t][j] y[position of slot (t, j)] in fp64 over the local slots."""
    S = len(ss)
    pos = np.full(T * k, -1, np.int64)
    pos[ss] = np.arange(S)
    pos = pos.reshape(T, k)
    out = np.zeros((T, D), np.float64)
    wf = w.astype(np.float64)
    for j in range(k):
        m = pos[:, j] >= 0
        out[m] += wf[m, j:j + 1] * y[pos[m, j]].astype(np.float64)
    return out


# (workload, moe_forward flags): the twelve workloads on their default routes, and the
# skewed MXFP8 workload once more with exact sums (the bf16 expansion) for comparison
CASES = [(i, 0) for i in range(1, 13)] + [(4, moe.FLAG_EXACT_SUMS)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("i,flags", CASES,
                         ids=[synth.WORKLOADS[i].name + ("-exact" if f else "") for i, f in CASES])
def test_fullsize_workload(i, flags):
    t_start = time.perf_counter()
    wl = synth.WORKLOADS[i]
    fmt, T, D, F, E, k = wl.fmt, wl.T, wl.D, wl.F, wl.E, wl.k
    eb, ee = wl.e_begin, wl.local_end
    nv, a16, f8 = fmt == "nvfp4", fmt in ("w4a16", "bf16"), fmt == "fp8"
    report("fullsize", workload=wl.name, T=T, D=D, F=F, E=E, local=f"[{eb},{ee})")
    h, wr, bias = wl.hidden(), wl.router_weight(), wl.router_bias()
    d_h, d_wr = to_dev(h), to_dev(wr)
    d_bias = None if bias is None else to_dev(bias)
    gu, dn = device_weights(wl)

    # ---- router, all tokens (the bench's call)
    ws = moe.route_workspace(T, D, E)
    idx, w, _, amax = moe.route(d_h, d_wr, k, d_bias, want_amax=nv, workspace=ws)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route(h, wr, k=k, bias=bias)
    assert np.array_equal(host(idx), o_idx), "top-k indices differ"
    np.testing.assert_allclose(host(w), o_w, rtol=1e-6, atol=0)
    if nv:
        assert host(amax)[0] == np.abs(synth.bf16_to_f32(h)).max()

    # ---- forward with taps (the bench's layer)
    layer = moe.Layer(fmt, T, D, F, E, gu, dn, top_k=k, e_begin=eb, e_end=ee, flags=flags)
    native8 = scaled_fp8(layer)
    inter_tol = INTER_TOL_SCALED_FP8 if native8 else INTER_TOL_EXACT
    report("  plan", **layer.plan())
    layer.enable_taps()
    out = host(layer.forward(d_h, idx, w, h_amax=amax))
    torch.cuda.synchronize()
    tp = {name: host(t) for name, t in layer.taps.items()}
    del layer

    # permutation
    counts, offsets, ss = oracle.permute(o_idx, eb, ee)
    S = int(offsets[-1])
    assert np.array_equal(tp["counts"], counts) and np.array_equal(tp["offsets"], offsets)
    assert np.array_equal(tp["sorted_slot"][:S], ss), "sorted slot order differs"

    # hidden-state codes (all tokens) and the exact activation values of every token
    hf = synth.bf16_to_f32(h)
    a_ts = a_rs = None
    if nv:
        a_c, a_s, a_ts = oracle.quant_nvfp4(hf)
        assert np.float32(tp["a_tscale"][0]) == a_ts
    elif f8:
        a_c, a_rs = oracle.quant_fp8_rows(hf)
        assert np.array_equal(tp["a_tscale"].view(np.uint32), a_rs.view(np.uint32)), "hidden row scales differ"
    elif not a16:
        a_c, a_s = oracle.quant_mxfp4(hf) if fmt == "mxfp4" else oracle.quant_mxfp8(hf)
    if a16:  # W4A16 and bf16 experts keep the hidden states in bf16
        act = hf.astype(np.float64)
    elif f8:
        assert np.array_equal(tp["a_codes"], a_c), "hidden codes differ"
        act = oracle.dequant_fp8_rows(a_c)
    else:
        assert np.array_equal(tp["a_codes"], a_c) and np.array_equal(tp["a_scales"], a_s), "hidden codes differ"
        act = _dequant(fmt, a_c, a_s)
    del hf

    # intermediate codes given the GPU's fp32 values (all S rows)
    g_inter = tp["inter"][:S]
    g_codes = tp["inter_codes"][:S]
    g_scales = tp["inter_scales"][:S] if "inter_scales" in tp else None
    if f8:  # the fp32 row scales
        g_scales = tp["inter_tscale"][:S]
    g_its = tp["inter_tscale"][0] if nv else None
    check_intermediate_codes(fmt, g_inter, g_codes, g_scales, g_its)
    g_y = tp["y"][:S]

    # ---- every touched expert: packed bytes, SwiGLU intermediate and y stage-wise
    inter_ref = np.empty((S, F), np.float32)
    y_stage = np.empty((S, D), np.float32)
    down_of = {}        # expert -> the oracle's down weights (for the independent pass)
    experts = {}        # expert -> (gate_up, down) of the oracle, decode workloads 1 and 2
    keep_gate_up = i in (1, 2, 11) and not flags
    worst_inter = worst_y = 0.0
    live = np.nonzero(counts)[0]
    for n_done, el in enumerate(live):
        e = eb + int(el)
        p0, p1 = int(offsets[el]), int(offsets[el + 1])
        o_gu, o_dn = _oracle_expert(wl, e)
        for dev_w, ref in ((gu, o_gu), (dn, o_dn)):
            if fmt == "bf16":
                assert np.array_equal(untile(host(dev_w.codes[e:e + 1])),
                                      ref["codes"].view(np.uint8).reshape(1, ref["codes"].shape[1], -1)), \
                    f"expert {e} weights differ"
                continue
            assert np.array_equal(untile(host(dev_w.codes[e:e + 1])), ref["codes"]), f"expert {e} codes differ"
            if f8:
                assert np.array_equal(host(dev_w.tensor_scale[e:e + 1]).view(np.uint32),
                                      ref["tensor_scale"].view(np.uint32)), f"expert {e} channel scales differ"
                continue
            assert np.array_equal(untile(host(dev_w.scales[e:e + 1])), ref["scales"]), f"expert {e} scales differ"
            if nv or fmt == "w4a16":
                assert host(dev_w.tensor_scale[e:e + 1])[0] == ref["tensor_scale"][0]
        down_of[e] = o_dn
        if keep_gate_up:
            experts[e] = (o_gu, o_dn)
        wg, wd = _values(fmt, o_gu), _values(fmt, o_dn)
        tok = ss[p0:p1] // k
        # exact products, fp64 sums, rounded to fp32, then the format's scales
        g = _scale_sums(fmt, act[tok] @ wg.T, o_gu, None if a_rs is None else a_rs[tok], a_ts)
        gate, up = g[:, :F].astype(np.float64), g[:, F:].astype(np.float64)
        inter_ref[p0:p1] = (gate * up / (1.0 + np.exp(-gate))).astype(np.float32)
        gs = None if g_scales is None else g_scales[p0:p1]
        y = _scale_sums(fmt, _inter_values(fmt, g_codes[p0:p1], None if f8 else gs) @ wd.T, o_dn, gs, g_its)
        y_stage[p0:p1] = y
        scale_i = float(np.abs(inter_ref[p0:p1]).max())
        e_inter = float(np.abs(g_inter[p0:p1] - inter_ref[p0:p1]).max()) / max(scale_i, 1e-30)
        e_y = float(np.abs(g_y[p0:p1] - y).max()) / max(rms(y), 1e-30)
        worst_inter, worst_y = max(worst_inter, e_inter), max(worst_y, e_y)
        assert e_inter < inter_tol, f"expert {e}: SwiGLU intermediate differs by {e_inter:.2e} of its max"
        assert e_y <= 2e-3, f"expert {e}: down projection differs by {e_y:.2e} x RMS"
        if (n_done + 1) % 32 == 0:
            report("  progress", experts=f"{n_done + 1}/{len(live)}", s=f"{time.perf_counter() - t_start:.0f}")
    del act
    report("  experts", touched=len(live), slots=S, worst_inter_rel=f"{worst_inter:.2e}",
           worst_y_stage_over_rms=f"{worst_y:.2e}")

    # ---- combine alone (from the GPU's own y) and the output stage-wise
    wf = host(w)
    e_comb = float(np.abs(out - _combine(T, D, k, ss, wf, g_y)).max()) / max(rms(out), 1e-30)
    assert e_comb <= 2e-3, f"combine differs by {e_comb:.2e} x RMS"
    out_stage = _combine(T, D, k, ss, wf, y_stage)
    r_stage = rms(out_stage)
    e_stage = float(np.abs(out - out_stage).max()) / r_stage
    assert e_stage <= 2e-3, f"stage-wise output error {e_stage:.2e} x RMS"
    has_local = ((o_idx >= eb) & (o_idx < ee)).any(1)
    assert not out[~has_local].any(), "tokens without a local slot must be zero"

    # ---- the output fully independently: the oracle quantises the reference intermediate
    if fmt in ("w4a16", "bf16"):
        i_codes, i_scales, i_ts = oracle.round_bf16(inter_ref), None, None
    elif nv:
        i_codes, i_scales, i_ts = oracle.quant_nvfp4(inter_ref)
    elif fmt == "mxfp4":
        (i_codes, i_scales), i_ts = oracle.quant_mxfp4(inter_ref), None
    elif f8:  # i_scales: the row scales [S]
        (i_codes, i_scales), i_ts = oracle.quant_fp8_rows(inter_ref), None
    else:
        (i_codes, i_scales), i_ts = oracle.quant_mxfp8(inter_ref), None
    rows_c, flips = _code_flips(fmt, g_codes, i_codes)
    rows_s = np.zeros(S, bool) if i_scales is None else (g_scales.reshape(S, -1) != i_scales.reshape(S, -1)).any(1)
    ts_same = (not nv) or np.float32(g_its) == np.float32(i_ts)
    flipped = rows_c | rows_s if ts_same else np.ones(S, bool)
    y_ind = y_stage.copy()
    for el in live:
        e = eb + int(el)
        p0, p1 = int(offsets[el]), int(offsets[el + 1])
        sel = np.nonzero(flipped[p0:p1])[0] + p0
        if len(sel) == 0:
            continue
        o_dn = down_of[e]
        isc = None if i_scales is None else i_scales[sel]
        y_ind[sel] = _scale_sums(fmt, _inter_values(fmt, i_codes[sel], None if f8 else isc) @ _values(fmt, o_dn).T,
                                 o_dn, isc, i_ts)
    out_ind = _combine(T, D, k, ss, wf, y_ind)
    r_ind = rms(out_ind)
    bad_tok = np.zeros(T, bool)
    bad_tok[ss[flipped] // k] = True
    err = np.abs(out - out_ind).max(1) / r_ind
    e_clean = float(err[~bad_tok].max()) if (~bad_tok).any() else 0.0
    e_flipped = float(err[bad_tok].max()) if bad_tok.any() else 0.0
    rel_rms = float(np.sqrt(np.mean((out - out_ind) ** 2))) / r_ind
    report("  flips", workload=wl.name + ("-exact" if flags else ""), elements=S * F, code_flips=flips,
           scale_flips=int(rows_s.sum()), tensor_scale_same=ts_same, rows_with_flips=int(flipped.sum()),
           tokens_with_flips=int(bad_tok.sum()), tokens=T)
    report("  output", stage_err=f"{e_stage:.2e}", independent_clean_err=f"{e_clean:.2e}",
           independent_flipped_tokens_err=f"{e_flipped:.2e}", independent_rel_rms=f"{rel_rms:.2e}",
           combine_err=f"{e_comb:.2e}")
    bounds = output_bounds(native8)
    assert flips <= bounds["max_flip_frac"] * S * F, f"{flips} intermediate code flips in {S * F} elements"
    assert e_clean <= 2e-3, f"independent output error {e_clean:.2e} x RMS on tokens without flips"
    assert rel_rms <= bounds["max_rel_rms"], f"independent output RMS error {rel_rms:.2e} x RMS"

    # ---- decode NVFP4 / MXFP8: the oracle's own forward on the experts the batch touches
    if keep_gate_up:
        used = np.array(sorted(experts))
        remap = np.full(E, -1, np.int32)
        remap[used] = np.arange(len(used), dtype=np.int32)
        cidx = remap[o_idx]
        cat = lambda key, j: np.concatenate([experts[int(e)][j][key] for e in used])
        o_gu = {key: None if experts[int(used[0])][0][key] is None else cat(key, 0)
                for key in ("codes", "scales", "tensor_scale")}
        o_dn = {key: None if experts[int(used[0])][1][key] is None else cat(key, 1)
                for key in ("codes", "scales", "tensor_scale")}
        t0 = time.perf_counter()
        ref, otp = oracle.moe_forward(fmt, h, cidx, o_w, D=D, F=F, E=len(used), taps=True, gate_up=o_gu,
                                      down=o_dn)
        t_orc = time.perf_counter() - t0
        o_isc = otp["inter_tscale"] if f8 else otp.get("inter_scales")
        e_s, e_i, fl, excl = check_outputs(fmt, out, ref, cidx, o_w, g_codes, g_scales, g_its, otp["inter_codes"],
                                           o_isc, ss, o_dn, D=D, F=F, E=len(used), e_begin=0,
                                           e_end=len(used), **output_bounds(native8))
        inter_vs_oracle = float(np.abs(otp["inter"] - inter_ref).max()) / float(np.abs(inter_ref).max())
        report("  oracle forward", seconds=f"{t_orc:.1f}", stage_err=f"{e_s:.2e}", independent_err=f"{e_i:.2e}",
               code_flips=fl, tokens_with_flips=excl, composed_vs_oracle_inter=f"{inter_vs_oracle:.1e}")
        assert inter_vs_oracle < 1e-6
    report("  done", seconds=f"{time.perf_counter() - t_start:.0f}")
