"""GPU parity at the full sizes of the ten benchmarked workloads, through the same calls
and launch configuration that bench.py times (moe.route + moe.Layer.forward).

Whole-batch, bit-exact: top-k indices of every token, max |h|, the permutation, every
hidden-state code and scale, and every intermediate code and scale given the GPU's own
fp32 intermediate. The oracle cannot run the full layer at these sizes in seconds, so
the expert arithmetic is checked on sampled rows of three local experts (the hottest,
the median and the coldest non-empty one): packed weight bytes bit-exact, the fp32
SwiGLU intermediate against an fp64 recomputation from the oracle's quantised weights
and the verified hidden-state codes, and the per-slot down projection y stage-wise from
the GPU's intermediate codes. The combine is checked on every token from the per-slot
y: out[t] = sum_j w[t][j] y[slot(t, j)] in fp64.
"""
import numpy as np
import pytest
import torch

import block_scaled_moe_amd as moe
import oracle
import synth
from gpu_util import check_intermediate_codes, device_weights, host, report, rms, to_dev, untile

pytestmark = pytest.mark.gpu

ROWS_PER_EXPERT = 16


def _dequant_mx(fmt, codes, scales):
    return oracle.dequant_mxfp4(codes, scales) if fmt == "mxfp4" else oracle.dequant_mxfp8(codes, scales)


def _expert_reference(wl, e, a_rows, a_ts, inter_codes, inter_scales, inter_ts):
    """fp64 gate_up -> SwiGLU (rounded to fp32) of the given dequantised hidden rows, and
    the down projection of the given intermediate codes, for expert e (oracle weights)."""
    nv = wl.fmt == "nvfp4"
    a16 = wl.fmt == "w4a16"
    F = wl.F
    if wl.fmt == "bf16":  # unquantised weights: the masters are the packed values
        gm, dm = wl.gate_up_master(e), wl.down_master(e)
        wg, wd = synth.bf16_to_f32(gm[0]).astype(np.float64), synth.bf16_to_f32(dm[0]).astype(np.float64)
        ai = synth.bf16_to_f32(np.asarray(inter_codes).view(np.uint16)).astype(np.float64)
        g = (a_rows @ wg.T).astype(np.float32)
        gate, up = g[:, :F].astype(np.float64), g[:, F:].astype(np.float64)
        inter = (gate * up / (1.0 + np.exp(-gate))).astype(np.float32)
        y = (ai @ wd.T).astype(np.float32)
        return {"codes": gm.view(np.uint8).reshape(1, gm.shape[1], -1)}, \
               {"codes": dm.view(np.uint8).reshape(1, dm.shape[1], -1)}, inter, y
    gu = oracle.quantize_weights(wl.fmt, wl.gate_up_master(e))
    dn = oracle.quantize_weights(wl.fmt, wl.down_master(e))
    if nv:
        wg = oracle.dequant_nvfp4(gu["codes"][0], gu["scales"][0], 1.0, with_tensor=False)
        wd = oracle.dequant_nvfp4(dn["codes"][0], dn["scales"][0], 1.0, with_tensor=False)
        s_gu = np.float32(np.float32(a_ts) * gu["tensor_scale"][0])
        s_dn = np.float32(np.float32(inter_ts) * dn["tensor_scale"][0])
        ai = oracle.dequant_nvfp4(inter_codes, inter_scales, 1.0, with_tensor=False)
    elif a16:
        wg = oracle.dequant_nvfp4(gu["codes"][0], gu["scales"][0], 1.0, with_tensor=False)
        wd = oracle.dequant_nvfp4(dn["codes"][0], dn["scales"][0], 1.0, with_tensor=False)
        s_gu, s_dn = np.float32(gu["tensor_scale"][0]), np.float32(dn["tensor_scale"][0])
        ai = synth.bf16_to_f32(np.asarray(inter_codes).view(np.uint16)).astype(np.float64)
    else:
        wg = _dequant_mx(wl.fmt, gu["codes"][0], gu["scales"][0])
        wd = _dequant_mx(wl.fmt, dn["codes"][0], dn["scales"][0])
        ai = _dequant_mx(wl.fmt, inter_codes, inter_scales)
    acc = a_rows @ wg.T                       # exact products, fp64 sums
    g = acc.astype(np.float32)
    if nv or a16:
        g = (g * s_gu).astype(np.float32)     # fl32(fl32(sum) * fl32(s_a * s_w)), W4A16 s_w alone
    gate, up = g[:, :F].astype(np.float64), g[:, F:].astype(np.float64)
    inter = (gate * up / (1.0 + np.exp(-gate))).astype(np.float32)
    y = (ai @ wd.T).astype(np.float32)
    if nv or a16:
        y = (y * s_dn).astype(np.float32)
    return gu, dn, inter, y


@pytest.mark.timeout(900)
@pytest.mark.parametrize("i", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10], ids=lambda i: synth.WORKLOADS[i].name)
def test_fullsize_workload(i):
    wl = synth.WORKLOADS[i]
    T, D, F, E, k = wl.T, wl.D, wl.F, wl.E, wl.k
    eb, ee = wl.e_begin, wl.local_end
    nv = wl.fmt == "nvfp4"
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
    layer = moe.Layer(wl.fmt, T, D, F, E, gu, dn, top_k=k, e_begin=eb, e_end=ee)
    layer.enable_taps()
    out = host(layer.forward(d_h, idx, w, h_amax=amax))
    torch.cuda.synchronize()
    tp = {name: host(t) for name, t in layer.taps.items()}

    # permutation
    counts, offsets, ss = oracle.permute(o_idx, eb, ee)
    S = int(offsets[-1])
    assert np.array_equal(tp["counts"], counts) and np.array_equal(tp["offsets"], offsets)
    assert np.array_equal(tp["sorted_slot"][:S], ss), "sorted slot order differs"

    # hidden-state codes (all tokens)
    hf = synth.bf16_to_f32(h)
    a16 = wl.fmt in ("w4a16", "bf16")
    a_ts = None
    if nv:
        a_c, a_s, a_ts = oracle.quant_nvfp4(hf)
        assert np.float32(tp["a_tscale"][0]) == a_ts
    elif not a16:
        a_c, a_s = oracle.quant_mxfp4(hf) if wl.fmt == "mxfp4" else oracle.quant_mxfp8(hf)
    if not a16:  # W4A16 keeps the hidden states in bf16
        assert np.array_equal(tp["a_codes"], a_c) and np.array_equal(tp["a_scales"], a_s), "hidden codes differ"

    # intermediate codes given the GPU's fp32 values (all S rows)
    i_ts = tp["inter_tscale"][0] if nv else None
    i_sc = tp["inter_scales"] if "inter_scales" in tp else None
    check_intermediate_codes(wl.fmt, tp["inter"][:S], tp["inter_codes"][:S], None if i_sc is None else i_sc[:S], i_ts)

    # ---- expert arithmetic on sampled rows of three experts
    live = np.nonzero(counts)[0]
    order = live[np.argsort(counts[live], kind="stable")]
    for el in sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])}):
        e = eb + el
        p0, p1 = int(offsets[el]), int(offsets[el + 1])
        rows = np.unique(np.linspace(p0, p1 - 1, min(ROWS_PER_EXPERT, p1 - p0)).round().astype(np.int64))
        tok = ss[rows] // k
        if a16:
            a_rows = hf[tok].astype(np.float64)
        elif nv:
            a_rows = oracle.dequant_nvfp4(a_c[tok], a_s[tok], 1.0, with_tensor=False)
        else:
            a_rows = _dequant_mx(wl.fmt, a_c[tok], a_s[tok])
        o_gu, o_dn, inter_ref, y_ref = _expert_reference(wl, e, a_rows, a_ts, tp["inter_codes"][rows],
                                                         None if i_sc is None else i_sc[rows], i_ts)
        # packed weights of this expert, bit-exact after undoing the tiling
        for dev_w, ref in ((gu, o_gu), (dn, o_dn)):
            assert np.array_equal(untile(host(dev_w.codes[e:e + 1])), ref["codes"]), f"expert {e} codes differ"
            if "scales" in ref:
                assert np.array_equal(untile(host(dev_w.scales[e:e + 1])), ref["scales"]), f"expert {e} scales differ"
        inter_err = float(np.abs(tp["inter"][rows] - inter_ref).max()) / float(np.abs(inter_ref).max())
        y_err = float(np.abs(tp["y"][rows] - y_ref).max()) / rms(y_ref)
        report("  expert", e=e, rows=f"{len(rows)} of {p1 - p0}", inter_rel=f"{inter_err:.2e}",
               y_err_over_rms=f"{y_err:.2e}")
        assert inter_err < 1e-5, f"expert {e}: SwiGLU intermediate differs by {inter_err:.2e} of its max"
        assert y_err <= 2e-3, f"expert {e}: down projection differs by {y_err:.2e} x RMS"

    # ---- combine, every token, from the per-slot y
    pos = np.full(T * k, -1, np.int64)
    pos[ss] = np.arange(S)
    pos = pos.reshape(T, k)
    ref = np.zeros((T, D), np.float64)
    wf = host(w).astype(np.float64)
    for j in range(k):
        m = pos[:, j] >= 0
        ref[m] += wf[m, j:j + 1] * tp["y"][pos[m, j]].astype(np.float64)
    err = float(np.abs(out - ref).max()) / rms(ref)
    report("  combine", err_over_rms=f"{err:.2e}")
    assert err <= 2e-3, f"combine differs by {err:.2e} x RMS"
