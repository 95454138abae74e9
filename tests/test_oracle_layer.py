"""Oracle router, permutation and MoE layer pinned against library routines,
a textbook fp64 MoE (BLAS matmul), brute force and invariants.

Routing: eight of 384 routed experts per token, no shared expert (vLLM recipe
"thinkingmachines/Inkling-2-Small", section "Overview"; AI Primer section "NVFP4
and MXFP8 experts"). Expert parallelism shards experts (recipe "Overview").
"""
import numpy as np
import pytest
import scipy.special

import oracle
import synth

f32 = np.float32


def _small(fmt="nvfp4", T=24, D=64, F=32, E=16, seed=3, skew=False):
    wl = synth.custom(fmt, T=T, D=D, F=F, E=E, seed=seed, skew=skew)
    return wl, wl.hidden(), wl.router_weight(), wl.router_bias()


# ------------------------------------------------------------------ router
def test_router_logits_are_sequential_fp32_sums():
    wl, h, wr, _ = _small(T=8, D=200, E=12)
    bias = np.linspace(-1, 1, 12).astype(f32)
    idx, w, lg = oracle.route(h, wr, k=4, bias=bias, want_logits=True)
    h32, w32 = synth.bf16_to_f32(h), synth.bf16_to_f32(wr)
    for t in range(8):
        for e in range(12):
            # numpy's add.accumulate is a strictly sequential fp32 running sum
            ref = np.add.accumulate(h32[t] * w32[e], dtype=f32)[-1] + bias[e]
            assert lg[t, e] == f32(ref)


def test_router_topk_order_ties_and_weights():
    wl, h, wr, _ = _small(T=64, D=64, E=40)
    wr = wr.copy()
    wr[7] = wr[3]      # experts 3 and 7 always tie
    wr[20] = wr[9]     # experts 9 and 20 always tie
    idx, w, lg = oracle.route(h, wr, k=8, want_logits=True)
    for t in range(64):
        order = np.lexsort((np.arange(40), -lg[t].astype(np.float64)))[:8]
        assert list(idx[t]) == list(order)
        ref = scipy.special.softmax(lg[t, order].astype(np.float64))
        np.testing.assert_allclose(w[t], ref, rtol=2e-7)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6
        assert np.all(np.diff(w[t]) <= 0)
        sel = set(idx[t].tolist())
        if 3 in sel and 7 in sel:
            assert list(idx[t]).index(3) < list(idx[t]).index(7)
        if 7 in sel:
            assert 3 in sel  # 3 ranks with 7 and wins the tie


def test_router_weights_equal_full_softmax_renormalised():
    wl, h, wr, _ = _small(T=16, D=128, E=64)
    idx, w, lg = oracle.route(h, wr, k=8, want_logits=True)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=2e-7)


def test_skew_bias_concentrates_routing():
    wl = synth.custom("mxfp8", T=2048, D=128, F=32, E=384, skew=True, seed=4)
    idx, w = oracle.route(wl.hidden(), wl.router_weight(), k=8, bias=wl.router_bias())
    counts = np.bincount(idx.reshape(-1), minlength=384)
    hottest = int(np.argmax(wl.router_bias()))
    assert counts.argmax() == hottest
    assert counts[hottest] > 0.9 * 2048      # nearly every token picks the rank-1 expert
    assert (counts > 0).sum() < 300          # the cold tail is mostly untouched


# ------------------------------------------------------------------ permutation
def test_permute_is_stable_counting_sort():
    rng = np.random.default_rng(0)
    idx = np.stack([rng.permutation(50)[:8] for _ in range(37)]).astype(np.int32)
    for eb, ee in ((0, 50), (10, 23), (49, 50)):
        counts, offs, ss = oracle.permute(idx, eb, ee)
        flat = idx.reshape(-1)
        local = np.nonzero((flat >= eb) & (flat < ee))[0]
        ref = local[np.argsort(flat[local], kind="stable")]
        assert np.array_equal(ss, ref)
        assert np.array_equal(counts, np.bincount(flat[local] - eb, minlength=ee - eb))
        assert offs[0] == 0 and np.array_equal(np.diff(offs), counts)
        assert sorted(ss.tolist()) == sorted(local.tolist())


# ------------------------------------------------------------------ layer
def _textbook_moe(h, gu, dn, idx, w, F, e_range=None):
    """Textbook MoE in fp64 with library matmuls: out[t] = sum_j w_tj * down(SwiGLU(gate_up(h_t)))."""
    H = synth.bf16_to_f32(h).astype(np.float64)
    out = np.zeros((H.shape[0], dn.shape[1]))
    for t in range(H.shape[0]):
        for j in range(idx.shape[1]):
            e = idx[t, j]
            if e_range and not (e_range[0] <= e < e_range[1]):
                continue
            W = synth.bf16_to_f32(gu[e]).astype(np.float64)
            g, u = W[:F] @ H[t], W[F:] @ H[t]
            a = g * u / (1.0 + np.exp(-g))
            out[t] += w[t, j] * (synth.bf16_to_f32(dn[e]).astype(np.float64) @ a)
    return out


def test_unquantised_layer_equals_textbook_moe():
    wl, h, wr, _ = _small(T=12, D=64, F=32, E=16)
    gu, dn = wl.gate_up_master(0, 16), wl.down_master(0, 16)
    idx, w = oracle.route(h, wr, k=8)
    out = oracle.moe_forward("none", h, idx, w, D=64, F=32, E=16, gate_up_master=gu, down_master=dn)
    ref = _textbook_moe(h, gu, dn, idx, w, 32)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())


def _quantised(fmt, wl):
    E = wl.E
    return (oracle.quantize_weights(fmt, wl.gate_up_master(0, E)),
            oracle.quantize_weights(fmt, wl.down_master(0, E)))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4"])
def test_quantised_layer_composes_from_pinned_parts(fmt):
    """The C pipeline equals a numpy composition of the (pinned) quantisers and BLAS matmuls."""
    T, D, F, E = 20, 64, 64, 12
    wl, h, wr, _ = _small(fmt, T=T, D=D, F=F, E=E, seed=8)
    gu, dn = _quantised(fmt, wl)
    idx, w = oracle.route(h, wr, k=8)
    out, tp = oracle.moe_forward(fmt, h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn, taps=True)
    H = synth.bf16_to_f32(h)
    mxq, mxd = (oracle.quant_mxfp4, oracle.dequant_mxfp4) if fmt == "mxfp4" else (oracle.quant_mxfp8,
                                                                                  oracle.dequant_mxfp8)
    if fmt == "nvfp4":
        ac, as_, ats = oracle.quant_nvfp4(H)
        A = oracle.dequant_nvfp4(ac, as_, ats, with_tensor=False)
    else:
        ac, as_ = mxq(H)
        A, ats = mxd(ac, as_), f32(1)
    assert np.array_equal(ac, tp["a_codes"]) and np.array_equal(as_, tp["a_scales"])
    counts, offs, ss = oracle.permute(idx, 0, E)
    S = len(ss)
    inter = np.zeros((S, F), f32)
    for p, s in enumerate(ss):
        t, e = s // 8, idx.reshape(-1)[s]
        if fmt == "nvfp4":
            W = oracle.dequant_nvfp4(gu["codes"][e], gu["scales"][e], 1.0, with_tensor=False)
            sc = f32(ats * gu["tensor_scale"][e])
            gl = (W @ A[t]).astype(f32) * sc
        else:
            W = mxd(gu["codes"][e], gu["scales"][e])
            gl = (W @ A[t]).astype(f32)
        g, u = gl[:F].astype(np.float64), gl[F:].astype(np.float64)
        inter[p] = (g * u / (1.0 + np.exp(-g))).astype(f32)
    np.testing.assert_array_equal(inter, tp["inter"])
    if fmt == "nvfp4":
        ic, is_, its = oracle.quant_nvfp4(inter)
        I = oracle.dequant_nvfp4(ic, is_, its, with_tensor=False)
    else:
        ic, is_ = mxq(inter)
        I, its = mxd(ic, is_), f32(1)
    assert np.array_equal(ic, tp["inter_codes"]) and np.array_equal(is_, tp["inter_scales"])
    ref = np.zeros((T, D))
    for p, s in enumerate(ss):
        t, j = divmod(int(s), 8)
        e = idx[t, j]
        if fmt == "nvfp4":
            Wd = oracle.dequant_nvfp4(dn["codes"][e], dn["scales"][e], 1.0, with_tensor=False)
            y = (Wd @ I[p]).astype(f32) * f32(its * dn["tensor_scale"][e])
        else:
            y = (mxd(dn["codes"][e], dn["scales"][e]) @ I[p]).astype(f32)
        np.testing.assert_array_equal(y, tp["y"][p])
        ref[t] += float(w[t, j]) * y.astype(np.float64)
    np.testing.assert_allclose(out, ref.astype(f32), rtol=1e-6, atol=1e-9)


def test_quantisation_error_ordering_against_unquantised():
    T, D, F, E = 32, 128, 64, 16
    errs = {}
    for fmt in ("nvfp4", "mxfp8", "mxfp4", "w4a16"):
        wl, h, wr, _ = _small(fmt, T=T, D=D, F=F, E=E, seed=12)
        gu_m, dn_m = wl.gate_up_master(0, E), wl.down_master(0, E)
        idx, w = oracle.route(h, wr, k=8)
        ref = oracle.moe_forward("none", h, idx, w, D=D, F=F, E=E, gate_up_master=gu_m, down_master=dn_m)
        gu, dn = oracle.quantize_weights(fmt, gu_m), oracle.quantize_weights(fmt, dn_m)
        out = oracle.moe_forward(fmt, h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn)
        errs[fmt] = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert errs["mxfp8"] < 0.08 and errs["nvfp4"] < 0.35 and errs["mxfp4"] < 0.45
    assert errs["mxfp8"] < errs["nvfp4"] / 2 and errs["nvfp4"] < errs["mxfp4"]
    # bf16 activations: only the weights' rounding is left; removing one of two independent
    # errors of similar size shrinks the total by about sqrt(2)
    assert errs["w4a16"] < errs["nvfp4"] / 1.25 and errs["w4a16"] < 0.25


@pytest.mark.parametrize("fmt", ["none", "mxfp8", "mxfp4", "w4a16"])
def test_expert_parallel_shares_add_up(fmt):
    """Four expert ranges (an EP4 split) sum to the full layer. NVFP4 is excluded:
    its intermediate tensor scale is taken over each share's own slots."""
    T, D, F, E = 16, 64, 32, 16
    wl, h, wr, _ = _small("mxfp8" if fmt == "none" else fmt, T=T, D=D, F=F, E=E, seed=21)
    idx, w = oracle.route(h, wr, k=8)
    kw = dict(D=D, F=F, E=E)
    if fmt == "none":
        kw.update(gate_up_master=wl.gate_up_master(0, E), down_master=wl.down_master(0, E))
    else:
        gu, dn = _quantised(fmt, wl)
        kw.update(gate_up=gu, down=dn)
    full = oracle.moe_forward(fmt, h, idx, w, **kw)
    parts = sum(oracle.moe_forward(fmt, h, idx, w, e_begin=4 * r, e_end=4 * r + 4, **kw).astype(np.float64)
                for r in range(4))
    np.testing.assert_allclose(parts, full, rtol=2e-6, atol=1e-6 * np.abs(full).max())


def test_local_share_zero_rows_and_token_subset():
    T, D, F, E = 40, 64, 32, 32
    wl, h, wr, _ = _small("nvfp4", T=T, D=D, F=F, E=E, seed=5)
    gu, dn = _quantised("nvfp4", wl)
    idx, w = oracle.route(h, wr, k=8)
    out = oracle.moe_forward("nvfp4", h, idx, w, D=D, F=F, E=E, e_begin=0, e_end=6, gate_up=gu, down=dn)
    has_local = ((idx >= 0) & (idx < 6)).any(1)
    assert not out[~has_local].any()
    assert np.abs(out[has_local]).min(1).max() > 0
    sub = np.array([3, 17, 31], np.int32)
    for fmt_ in ("nvfp4",):
        part = oracle.moe_forward(fmt_, h, idx, w, D=D, F=F, E=E, e_begin=0, e_end=6, gate_up=gu, down=dn,
                                  tok_list=sub)
        assert np.array_equal(part[sub], out[sub])
        rest = np.setdiff1d(np.arange(T), sub)
        assert not part[rest].any()


def test_empty_batch_is_a_no_op():
    wl, h, wr, _ = _small(T=4, D=64, F=32, E=16)
    gu, dn = _quantised("nvfp4", wl)
    out = oracle.moe_forward("nvfp4", h[:0], np.zeros((0, 8), np.int32), np.zeros((0, 8), f32),
                             D=64, F=32, E=16, gate_up=gu, down=dn)
    assert out.shape == (0, 64)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4", "w4a16"])
def test_down_combine_reproduces_the_forward(fmt):
    """The stage-wise entry point (down projection + combine from given intermediate codes),
    fed the forward's own intermediate codes, gives the forward's output bit for bit, also
    on an expert-parallel share."""
    T, D, F, E = 24, 64, 96, 12
    wl, h, wr, _ = _small(fmt, T=T, D=D, F=F, E=E, seed=44)
    gu, dn = _quantised(fmt, wl)
    idx, w = oracle.route(h, wr, k=8)
    for eb, ee in ((0, E), (3, 8)):
        out, tp = oracle.moe_forward(fmt, h, idx, w, D=D, F=F, E=E, e_begin=eb, e_end=ee, gate_up=gu, down=dn,
                                     taps=True)
        ts = tp["inter_tscale"][0] if fmt == "nvfp4" else None
        got = oracle.down_combine(fmt, idx, w, tp["inter_codes"], tp.get("inter_scales"), ts, dn, D=D, F=F, E=E,
                                  e_begin=eb, e_end=ee)
        assert np.array_equal(got.view(np.uint32), out.view(np.uint32))


# ------------------------------------------------------------------ W4A16
def _bf16_bits(x) -> np.ndarray:
    """torch's fp32 -> bf16 conversion (nearest, ties to even) as uint16 bit patterns."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, f32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_w4a16_composes_from_pinned_parts():
    """NVFP4 weights with bf16 activations (vLLM recipe "thinkingmachines/Inkling-Small",
    section "Variants": the weights dequantised on the fly): the C pipeline equals a numpy
    composition of the pinned NVFP4 dequantiser, BLAS matmuls on the unquantised bf16
    hidden states, the weight tensor scale on the fp32 sums, and torch's bf16 rounding of
    the SwiGLU output."""
    T, D, F, E = 20, 64, 64, 12
    wl, h, wr, _ = _small("nvfp4", T=T, D=D, F=F, E=E, seed=9)
    gu, dn = _quantised("w4a16", wl)
    idx, w = oracle.route(h, wr, k=8)
    out, tp = oracle.moe_forward("w4a16", h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn, taps=True)
    assert "a_codes" not in tp  # hidden states are not quantised
    H = synth.bf16_to_f32(h).astype(np.float64)
    counts, offs, ss = oracle.permute(idx, 0, E)
    S = len(ss)
    inter = np.zeros((S, F), f32)
    for p, s in enumerate(ss):
        t, e = s // 8, idx.reshape(-1)[s]
        W = oracle.dequant_nvfp4(gu["codes"][e], gu["scales"][e], 1.0, with_tensor=False)
        gl = (W @ H[t]).astype(f32) * f32(gu["tensor_scale"][e])
        g, u = gl[:F].astype(np.float64), gl[F:].astype(np.float64)
        inter[p] = (g * u / (1.0 + np.exp(-g))).astype(f32)
    np.testing.assert_array_equal(inter, tp["inter"])
    ib = _bf16_bits(inter)
    assert np.array_equal(ib, tp["inter_codes"])
    I = synth.bf16_to_f32(ib).astype(np.float64)
    ref = np.zeros((T, D))
    for p, s in enumerate(ss):
        t, j = divmod(int(s), 8)
        e = idx[t, j]
        Wd = oracle.dequant_nvfp4(dn["codes"][e], dn["scales"][e], 1.0, with_tensor=False)
        y = (Wd @ I[p]).astype(f32) * f32(dn["tensor_scale"][e])
        np.testing.assert_array_equal(y, tp["y"][p])
        ref[t] += float(w[t, j]) * y.astype(np.float64)
    np.testing.assert_allclose(out, ref.astype(f32), rtol=1e-6, atol=1e-9)


def _grid_masters(E, N, K, seed):
    """bf16 masters whose NVFP4 encoding is exact up to the tensor scale's rounding: every
    value is c * 2^-7 with c on the E2M1 grid, and every 16-block holds a +-6 (so each block
    and the tensor share amax 6 * 2^-7 and the block scale is E4M3's 448)."""
    rng = np.random.default_rng(seed)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    c = grid[rng.integers(0, 8, (E, N, K))] * rng.choice([-1.0, 1.0], (E, N, K))
    blocks = c.reshape(E, N, K // 16, 16)
    pos = rng.integers(0, 16, (E, N, K // 16))
    np.put_along_axis(blocks, pos[..., None], 6.0 * rng.choice([-1.0, 1.0], (E, N, K // 16, 1)), axis=3)
    return _bf16_bits((blocks.reshape(E, N, K) * 2.0 ** -7).astype(f32))


def test_w4a16_on_exactly_encodable_weights_is_the_bf16_layer():
    """When the NVFP4 weights reproduce the masters, W4A16 is the unquantised layer up to
    the bf16 rounding of the SwiGLU output (and ulp-level tensor-scale rounding), while
    W4A4 still carries the activation quantisation error."""
    T, D, F, E = 24, 128, 64, 12
    wl, h, wr, _ = _small("nvfp4", T=T, D=D, F=F, E=E, seed=14)
    gu_m, dn_m = _grid_masters(E, 2 * F, D, 1), _grid_masters(E, D, F, 2)
    idx, w = oracle.route(h, wr, k=8)
    ref = oracle.moe_forward("none", h, idx, w, D=D, F=F, E=E, gate_up_master=gu_m, down_master=dn_m)
    gu, dn = oracle.quantize_weights("nvfp4", gu_m), oracle.quantize_weights("nvfp4", dn_m)
    W = oracle.dequant_nvfp4(gu["codes"].reshape(-1, D // 2), gu["scales"].reshape(-1, D // 16),
                             float(gu["tensor_scale"][0]))
    np.testing.assert_allclose(W.reshape(E, 2 * F, D), synth.bf16_to_f32(gu_m), rtol=2e-7, atol=0)
    a16 = oracle.moe_forward("w4a16", h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn)
    a4 = oracle.moe_forward("nvfp4", h, idx, w, D=D, F=F, E=E, gate_up=gu, down=dn)
    err16 = np.linalg.norm(a16 - ref) / np.linalg.norm(ref)
    err4 = np.linalg.norm(a4 - ref) / np.linalg.norm(ref)
    assert err16 < 3e-3, err16      # bf16 rounding of the intermediate only (2^-9 relative)
    assert err4 > 10 * err16, (err4, err16)


# ------------------------------------------------------------------ bf16 experts
def test_bf16_experts_compose_from_library_routines():
    """bf16 experts (the checkpoint's BF16 variant, vLLM recipe "thinkingmachines/Inkling-Small",
    section "Variants"): a BLAS composition on the unquantised bf16 masters with the fp32
    rounding of each sum and torch's bf16 rounding of the SwiGLU output."""
    T, D, F, E = 20, 64, 64, 12
    wl, h, wr, _ = _small("nvfp4", T=T, D=D, F=F, E=E, seed=10)
    gu_m, dn_m = wl.gate_up_master(0, E), wl.down_master(0, E)
    idx, w = oracle.route(h, wr, k=8)
    out, tp = oracle.moe_forward("bf16", h, idx, w, D=D, F=F, E=E, gate_up_master=gu_m, down_master=dn_m,
                                 taps=True)
    H = synth.bf16_to_f32(h).astype(np.float64)
    counts, offs, ss = oracle.permute(idx, 0, E)
    inter = np.zeros((len(ss), F), f32)
    for p, s in enumerate(ss):
        t, e = s // 8, idx.reshape(-1)[s]
        gl = (synth.bf16_to_f32(gu_m[e]).astype(np.float64) @ H[t]).astype(f32)
        g, u = gl[:F].astype(np.float64), gl[F:].astype(np.float64)
        inter[p] = (g * u / (1.0 + np.exp(-g))).astype(f32)
    np.testing.assert_array_equal(inter, tp["inter"])
    ib = _bf16_bits(inter)
    assert np.array_equal(ib, tp["inter_codes"])
    I = synth.bf16_to_f32(ib).astype(np.float64)
    ref = np.zeros((T, D))
    for p, s in enumerate(ss):
        t, j = divmod(int(s), 8)
        y = (synth.bf16_to_f32(dn_m[idx[t, j]]).astype(np.float64) @ I[p]).astype(f32)
        np.testing.assert_array_equal(y, tp["y"][p])
        ref[t] += float(w[t, j]) * y.astype(np.float64)
    np.testing.assert_allclose(out, ref.astype(f32), rtol=1e-6, atol=1e-9)


def test_bf16_experts_match_w4a16_on_exactly_encodable_weights():
    """Where NVFP4 reproduces the masters, W4A16 and bf16 experts run the same arithmetic
    up to the ulp-level rounding of the NVFP4 tensor scale; both stay within the
    intermediate's bf16 rounding of the fp64 textbook layer."""
    T, D, F, E = 24, 128, 64, 12
    wl, h, wr, _ = _small("nvfp4", T=T, D=D, F=F, E=E, seed=15)
    gu_m, dn_m = _grid_masters(E, 2 * F, D, 3), _grid_masters(E, D, F, 4)
    idx, w = oracle.route(h, wr, k=8)
    kw = dict(D=D, F=F, E=E)
    b16 = oracle.moe_forward("bf16", h, idx, w, gate_up_master=gu_m, down_master=dn_m, **kw)
    gu, dn = oracle.quantize_weights("nvfp4", gu_m), oracle.quantize_weights("nvfp4", dn_m)
    a16 = oracle.moe_forward("w4a16", h, idx, w, gate_up=gu, down=dn, **kw)
    ref = oracle.moe_forward("none", h, idx, w, gate_up_master=gu_m, down_master=dn_m, **kw)
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    assert float(np.abs(b16 - a16).max()) / rms < 1e-4
    assert np.linalg.norm(b16 - ref) / np.linalg.norm(ref) < 3e-3


def test_bf16_experts_shares_and_stagewise():
    """Four expert ranges add up to the full layer, and the stage-wise entry point fed the
    forward's own bf16 intermediate reproduces it bit for bit."""
    T, D, F, E = 16, 64, 96, 16
    wl, h, wr, _ = _small("nvfp4", T=T, D=D, F=F, E=E, seed=23)
    gu_m, dn_m = wl.gate_up_master(0, E), wl.down_master(0, E)
    idx, w = oracle.route(h, wr, k=8)
    kw = dict(D=D, F=F, E=E, gate_up_master=gu_m, down_master=dn_m)
    full = oracle.moe_forward("bf16", h, idx, w, **kw)
    parts = sum(oracle.moe_forward("bf16", h, idx, w, e_begin=4 * r, e_end=4 * r + 4, **kw).astype(np.float64)
                for r in range(4))
    np.testing.assert_allclose(parts, full, rtol=2e-6, atol=1e-6 * np.abs(full).max())
    for eb, ee in ((0, E), (3, 9)):
        out, tp = oracle.moe_forward("bf16", h, idx, w, e_begin=eb, e_end=ee, taps=True, **kw)
        got = oracle.down_combine("bf16", idx, w, tp["inter_codes"], None, None, dn_m, D=D, F=F, E=E,
                                  e_begin=eb, e_end=ee)
        assert np.array_equal(got.view(np.uint32), out.view(np.uint32))
