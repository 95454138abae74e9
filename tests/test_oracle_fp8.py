"""Oracle FP8 format: E4M3 with one fp32 scale per row (dynamic per-token activation scales,
one scale per output channel of the weights), pinned by hand-worked rows, torch's E4M3
conversion, closed forms on exactly encodable inputs and the layer's invariants.

Format: vLLM recipe "thinkingmachines/Inkling-Small", the "fp8" entry of its variants
(E4M3 with dynamic per-token activation quantisation). The weights' per-channel scales and
the row scale amax / 448 are this library's reading of that entry.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

f32 = np.float32


def _e4m3_values():
    """Every finite non-negative E4M3 value (codes 0..126) from the bit fields."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


# ------------------------------------------------------------------ row quantiser
def test_fp8_rows_hand_worked():
    # amax 7 -> scale 7 / 448 = 2^-6; 7 -> 448 (0x7E), 3.5 -> 224 = 1.75 * 2^7 (0x76),
    # -1.75 -> -112 = -1.75 * 2^6 (0xEE), 0 -> 0x00, 2^-15 -> 2^-9 (smallest subnormal, 0x01),
    # 2^-16 -> half the smallest subnormal: a tie, to even (0x00)
    x = np.zeros((3, 8), f32)
    x[0, :6] = [7.0, 3.5, -1.75, 0.0, 2.0 ** -15, 2.0 ** -16]
    x[2, 3] = -3.0                 # amax 3 -> scale 3/448 (inexact), -3 -> -448 (0xFE)
    codes, scales = oracle.quant_fp8_rows(x)
    assert scales[0] == 2.0 ** -6
    assert list(codes[0, :6]) == [0x7E, 0x76, 0xEE, 0x00, 0x01, 0x00]
    assert scales[1] == 1.0 and not codes[1].any()            # zero row: scale 1, zero codes
    assert scales[2] == f32(3.0) / f32(448.0) and codes[2, 3] == 0xFE
    assert oracle.fp8_row_scale(7.0) == 2.0 ** -6 and oracle.fp8_row_scale(0.0) == 1.0


def test_fp8_rows_match_torch_e4m3_and_closed_form_scale():
    h = synth.bf16_to_f32(synth.normal_bf16(6, 1, 0, 64 * 512, 1.0)).reshape(64, 512)
    h[3] *= f32(2.0 ** -100)       # tiny row
    h[4] = 0.0                     # zero row
    h[5, 7] = 1e6                  # one outlier: most of the row underflows to subnormals
    codes, scales = oracle.quant_fp8_rows(h)
    amax = np.abs(h).max(1)
    want = np.where(amax > 0, amax / f32(448.0), f32(1.0)).astype(f32)
    assert np.array_equal(scales, want)
    q = (h / scales[:, None]).astype(f32)
    assert np.abs(q).max() < 464   # the quotient never leaves E4M3's rounding range
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # every non-zero row reaches the largest code at its maximum
    nz = amax > 0
    assert np.all((codes[nz] & 0x7F).max(1) == 0x7E)
    # |x - x_hat| <= half an E4M3 ulp (relative 2^-4) or half the subnormal step s * 2^-10
    xh = oracle.dequant_fp8_rows(codes, scales)
    err = np.abs(h.astype(np.float64) - xh)
    bound = np.maximum(np.abs(h) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound)
    np.testing.assert_array_equal(oracle.dequant_fp8_rows(codes), _e4m3_values()[codes & 0x7F]
                                  * np.where(codes & 0x80, -1.0, 1.0))


def test_fp8_weights_have_one_scale_per_output_channel():
    wl = synth.custom("fp8", T=4, D=64, F=32, E=3, seed=9)
    m = wl.gate_up_master(0, 3)
    q = oracle.quantize_weights("fp8", m)
    assert q["scales"] is None and q["tensor_scale"].shape == (3, 64)
    for e in range(3):
        c, s = oracle.quant_fp8_rows(synth.bf16_to_f32(m[e]))
        assert np.array_equal(q["codes"][e], c) and np.array_equal(q["tensor_scale"][e], s)


# ------------------------------------------------------------------ layer
def _small(T, D, F, E, seed):
    wl = synth.custom("fp8", T=T, D=D, F=F, E=E, seed=seed)
    return wl, wl.hidden(), wl.router_weight()


def test_fp8_layer_composes_from_pinned_parts():
    """The C pipeline equals a numpy composition of the (pinned) row quantiser and BLAS matmuls:
    gate/up sums rounded to fp32 times fl32(token scale * channel scale), SwiGLU, the
    intermediate quantised per slot row, down sums times fl32(row scale * channel scale)."""
    T, D, F, E = 20, 64, 64, 12
    wl, h, wr = _small(T, D, F, E, 8)
    gu, dn = oracle.quantize_weights("fp8", wl.gate_up_master(0, E)), oracle.quantize_weights("fp8", wl.down_master(0, E))
    idx, w = oracle.route(h, wr, k=8)
    out, tp = oracle.moe_forward("fp8", h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn, taps=True)
    ac, ats = oracle.quant_fp8_rows(synth.bf16_to_f32(h))
    assert np.array_equal(ac, tp["a_codes"]) and np.array_equal(ats, tp["a_tscale"])
    A = oracle.dequant_fp8_rows(ac)
    _, _, ss = oracle.permute(idx, 0, E)
    S = len(ss)
    inter = np.zeros((S, F), f32)
    for p, s in enumerate(ss):
        t, e = s // 8, idx.reshape(-1)[s]
        sums = (oracle.dequant_fp8_rows(gu["codes"][e]) @ A[t]).astype(f32)
        gl = sums * (ats[t] * gu["tensor_scale"][e]).astype(f32)
        g, u = gl[:F].astype(np.float64), gl[F:].astype(np.float64)
        inter[p] = (g * u / (1.0 + np.exp(-g))).astype(f32)
    np.testing.assert_array_equal(inter, tp["inter"])
    ic, irs = oracle.quant_fp8_rows(inter)
    assert np.array_equal(ic, tp["inter_codes"]) and np.array_equal(irs, tp["inter_tscale"])
    I = oracle.dequant_fp8_rows(ic)
    ref = np.zeros((T, D))
    for p, s in enumerate(ss):
        t, j = divmod(int(s), 8)
        e = idx[t, j]
        y = (oracle.dequant_fp8_rows(dn["codes"][e]) @ I[p]).astype(f32) * (irs[p] * dn["tensor_scale"][e]).astype(f32)
        np.testing.assert_array_equal(y, tp["y"][p])
        ref[t] += float(w[t, j]) * y.astype(np.float64)
    np.testing.assert_allclose(out, ref.astype(f32), rtol=1e-6, atol=1e-9)


def _encodable_rows(shape, seed):
    """bf16 rows whose FP8 row encoding is exact: values c * 2^(j - 6) with c an E4M3 value,
    a +-448 in every row (so the row scale is the power of two 2^(j - 6)), and j varying
    from row to row in [-2, 2] so that every row (channel, token) has its own scale."""
    rng = np.random.default_rng(seed)
    vals = _e4m3_values()
    c = vals[rng.integers(0, 127, shape)] * rng.choice([-1.0, 1.0], shape)
    rows = c.reshape(-1, shape[-1])
    pos = rng.integers(0, shape[-1], rows.shape[0])
    rows[np.arange(rows.shape[0]), pos] = 448.0 * rng.choice([-1.0, 1.0], rows.shape[0])
    j = rng.integers(-2, 3, rows.shape[0]).astype(np.float64)
    x = (rows * np.exp2(j - 6)[:, None]).reshape(shape).astype(f32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), x


def test_fp8_on_exactly_encodable_inputs_is_the_unquantised_gate_up():
    """With hidden states and weights on the FP8 grid (power-of-two row scales, different per
    row), the SwiGLU output is fl32(SwiGLU(fl32(g), fl32(u))) of the exact fp64 sums of the
    masters, and the layer differs from the unquantised one only by the intermediate's
    rounding (3 mantissa bits: relative 2^-4 at most)."""
    T, D, F, E = 16, 128, 64, 8
    wl, _, wr = _small(T, D, F, E, 31)
    h, hx = _encodable_rows((T, D), 1)
    gu_m, gx = _encodable_rows((E, 2 * F, D), 2)
    dn_m, dx = _encodable_rows((E, D, F), 3)
    gu, dn = oracle.quantize_weights("fp8", gu_m), oracle.quantize_weights("fp8", dn_m)
    assert np.all(np.log2(gu["tensor_scale"]) == np.round(np.log2(gu["tensor_scale"])))
    assert len(np.unique(gu["tensor_scale"])) == 5
    idx, w = oracle.route(h, wr, k=8)
    out, tp = oracle.moe_forward("fp8", h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn, taps=True)
    _, _, ss = oracle.permute(idx, 0, E)
    H, G = hx.astype(np.float64), gx.astype(np.float64)
    for p, s in enumerate(ss):
        t, e = s // 8, idx.reshape(-1)[s]
        gl = (G[e] @ H[t]).astype(f32).astype(np.float64)   # exact fp64 sums (<= 44 bits)
        g, u = gl[:F], gl[F:]
        with np.errstate(over="ignore"):  # exp(-g) = inf for very negative g: SwiGLU 0
            want = (g * u / (1.0 + np.exp(-g))).astype(f32)
        np.testing.assert_allclose(tp["inter"][p], want, rtol=1.2e-7, atol=0)
    ref = oracle.moe_forward("none", h, idx, w, D=D, F=F, E=E, gate_up_master=gu_m, down_master=dn_m)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 2.0 ** -4 / np.sqrt(3), rel


def test_fp8_error_between_mxfp8_and_nvfp4():
    """Same 3 mantissa bits as MXFP8, so the same error scale; the fp32 row scale maps each
    row's maximum onto 448 exactly where MXFP8's power-of-two scale leaves a block maximum
    in [256, 512) and clips it above 448, which outweighs the coarser granularity on
    Gaussian rows of this width. Both stay well ahead of NVFP4."""
    T, D, F, E = 32, 128, 64, 16
    errs = {}
    for fmt in ("fp8", "mxfp8", "nvfp4"):
        wl = synth.custom(fmt, T=T, D=D, F=F, E=E, seed=12)
        h, wr = wl.hidden(), wl.router_weight()
        gu_m, dn_m = wl.gate_up_master(0, E), wl.down_master(0, E)
        idx, w = oracle.route(h, wr, k=8)
        ref = oracle.moe_forward("none", h, idx, w, D=D, F=F, E=E, gate_up_master=gu_m, down_master=dn_m)
        gu, dn = oracle.quantize_weights(fmt, gu_m), oracle.quantize_weights(fmt, dn_m)
        out = oracle.moe_forward(fmt, h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn)
        errs[fmt] = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert errs["mxfp8"] / 2 < errs["fp8"] < errs["mxfp8"] < errs["nvfp4"] / 2, errs


def test_fp8_expert_parallel_shares_add_up_and_down_combine():
    T, D, F, E = 16, 64, 32, 16
    wl, h, wr = _small(T, D, F, E, 21)
    gu, dn = oracle.quantize_weights("fp8", wl.gate_up_master(0, E)), oracle.quantize_weights("fp8", wl.down_master(0, E))
    idx, w = oracle.route(h, wr, k=8)
    kw = dict(D=D, F=F, E=E, gate_up=gu, down=dn)
    full = oracle.moe_forward("fp8", h, idx, w, **kw)
    parts = sum(oracle.moe_forward("fp8", h, idx, w, e_begin=4 * r, e_end=4 * r + 4, **kw).astype(np.float64)
                for r in range(4))
    np.testing.assert_allclose(parts, full, rtol=2e-6, atol=1e-6 * np.abs(full).max())
    for eb, ee in ((0, E), (3, 8)):
        out, tp = oracle.moe_forward("fp8", h, idx, w, e_begin=eb, e_end=ee, taps=True, **kw)
        got = oracle.down_combine("fp8", idx, w, tp["inter_codes"], None, tp["inter_tscale"], dn, D=D, F=F, E=E,
                                  e_begin=eb, e_end=ee)
        assert np.array_equal(got.view(np.uint32), out.view(np.uint32))
    # token subset: the wanted tokens' outputs are unchanged (row scales are per token)
    sub = np.array([1, 9, 14], np.int32)
    part = oracle.moe_forward("fp8", h, idx, w, tok_list=sub, **kw)
    assert np.array_equal(part[sub], full[sub]) and not np.delete(part, sub, 0).any()


@pytest.mark.parametrize("planted", ["up_scale_index", "slot_row_scale"])
def test_fp8_pins_catch_planted_mistakes(planted):
    """The composition pin above fails for plausible wiring mistakes: the up rows scaled by
    the gate rows' channel scales, or the intermediate rows' scales taken from the wrong slot."""
    T, D, F, E = 12, 64, 32, 12
    wl, h, wr = _small(T, D, F, E, 5)
    gu, dn = oracle.quantize_weights("fp8", wl.gate_up_master(0, E)), oracle.quantize_weights("fp8", wl.down_master(0, E))
    idx, w = oracle.route(h, wr, k=8)
    out, tp = oracle.moe_forward("fp8", h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn, taps=True)
    if planted == "up_scale_index":
        bad = dict(gu, tensor_scale=np.concatenate([gu["tensor_scale"][:, :F]] * 2, 1))
        mis = oracle.moe_forward("fp8", h, idx, w, D=D, F=F, E=E, gate_up=bad, down=dn, taps=True)[1]["inter"]
        assert not np.array_equal(mis, tp["inter"])
    else:
        rs = np.roll(tp["inter_tscale"], 1)
        mis = oracle.down_combine("fp8", idx, w, tp["inter_codes"], None, rs, dn, D=D, F=F, E=E)
        assert not np.allclose(mis, out, rtol=1e-3)
