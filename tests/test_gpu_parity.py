"""GPU path against the CPU oracle, through the C ABI (needs an MI355X).

Bit-exact: quantised weight codes, scales and tensor scales; router logits and top-k
indices; counts, offsets and the sorted slot order; hidden-state codes and scales;
the intermediate codes and scales given the GPU's own pre-quantisation values.
Within tolerance: gate weights (1e-6 relative), the SwiGLU intermediate, and the
layer output (max |error| <= 2e-3 x RMS of the oracle's output).
Sizes span several tiles in M, N and K with ragged tails; the layer cases cover both
formats, both tile shapes (decode and prefill), an expert-parallel share and skewed
routing.
"""
import numpy as np
import pytest
import torch

import block_scaled_moe_amd as moe
import oracle
import synth
from gpu_util import (INTER_TOL_EXACT, INTER_TOL_SCALED_FP8, case_inputs, check_intermediate_codes, check_outputs, host,
                      output_bounds, report, rms, scaled_fp8, to_dev, untile)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()


# ------------------------------------------------------------------ weights
def _adversarial_masters(E, N, K, seed):
    """bf16 masters with an all-zero expert, zero blocks, saturating and tiny values."""
    wl = synth.custom("nvfp4", T=1, D=K, F=N // 2, E=E, seed=seed)
    w = wl.gate_up_master(0, E).copy()
    w[0] = 0                                   # all-zero expert: tensor scale 1, all codes 0
    w[1, :, :32] = 0                           # zero blocks in a live expert
    w[1, 3, 5] = 0x8000                        # a negative zero
    big = synth.normal_bf16(seed, 9, 0, N * K, 300.0).reshape(N, K)
    w[E - 1] = big                             # large values (tensor scale >> 1)
    if E > 3:
        tiny = synth.normal_bf16(seed, 10, 0, N * K, 1e-6).reshape(N, K)
        w[2] = tiny                            # tiny values next to the live experts
    return w


def test_pack_bf16_weights_bitexact():
    """bf16 experts: the packing is a pure reordering into the tile layout."""
    w = _adversarial_masters(5, 256, 512, seed=8)
    got = moe.quantize_weights("bf16", to_dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(untile(host(got.codes)).view(np.uint16), w), "packed bf16 weights differ"


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4", "fp8"])
@pytest.mark.parametrize("shape", [(5, 256, 512), (2, 96, 2048)])
def test_quantize_weights_bitexact(fmt, shape):
    E, N, K = shape
    w = _adversarial_masters(E, N, K, seed=7)
    report("quantize_weights", fmt=fmt, E=E, N=N, K=K)
    got = moe.quantize_weights(fmt, to_dev(w))
    torch.cuda.synchronize()
    ref = oracle.quantize_weights(fmt, w)
    assert np.array_equal(untile(host(got.codes)), ref["codes"]), "codes differ"
    if fmt != "fp8":
        assert np.array_equal(untile(host(got.scales)), ref["scales"]), "scales differ"
    if fmt in ("nvfp4", "fp8"):  # FP8: the channel scales [E][N]
        assert np.array_equal(host(got.tensor_scale).view(np.uint32), ref["tensor_scale"].view(np.uint32))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4", "bf16", "fp8"])
@pytest.mark.parametrize("shape", [(3, 96, 512), (2, 256, 2048)])
def test_pack_rowmajor_checkpoint_bitexact(fmt, shape):
    """moe_pack_weights on the oracle's row-major quantisation (a pre-quantised checkpoint)
    gives the bytes moe_quantize_weights writes for the same masters, and untiles to it."""
    E, N, K = shape
    w = _adversarial_masters(E, N, K, seed=17)
    report("pack_weights", fmt=fmt, E=E, N=N, K=K)
    if fmt == "bf16":
        got = moe.pack_weights(fmt, to_dev(w))
    else:
        o = oracle.quantize_weights(fmt, w)
        ts = None if o["tensor_scale"] is None else to_dev(o["tensor_scale"])
        got = moe.pack_weights(fmt, to_dev(o["codes"]), None if o["scales"] is None else to_dev(o["scales"]), ts)
    ref = moe.quantize_weights(fmt, to_dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(host(got.codes), host(ref.codes)), "packed codes differ"
    assert np.array_equal(host(got.scales), host(ref.scales)), "packed scales differ"
    if fmt in ("nvfp4", "fp8"):
        assert np.array_equal(host(got.tensor_scale).view(np.uint32), host(ref.tensor_scale).view(np.uint32))
    if fmt == "bf16":
        assert np.array_equal(untile(host(got.codes)).view(np.uint16), w)
    elif fmt == "fp8":
        assert np.array_equal(untile(host(got.codes)), o["codes"])
        assert np.array_equal(host(got.tensor_scale).view(np.uint32), o["tensor_scale"].view(np.uint32))
    else:
        assert np.array_equal(untile(host(got.codes)), o["codes"]) and np.array_equal(untile(host(got.scales)),
                                                                                     o["scales"])


# ------------------------------------------------------------------ router
ROUTER_CASES = [
    dict(T=37, D=256, E=64, skew=False),      # exact path, ragged token tile
    dict(T=64, D=4096, E=384, skew=False),    # decode shape (exact path)
    dict(T=511, D=256, E=200, skew=False),    # largest exact-path batch, E not a multiple of 64
    dict(T=512, D=256, E=200, skew=False),    # smallest screened batch, padded expert tiles
    dict(T=1030, D=512, E=384, skew=True),    # screened, biased logits
    dict(T=8200, D=256, E=384, skew=False),   # screened, ragged tail
    dict(T=2048, D=4096, E=384, skew=True),   # screened at d_model 4096 with the skew bias
    dict(T=700, D=256, E=384, skew=False, k=4),                # screened, top-4
    dict(T=600, D=256, E=384, skew=False, adversarial=True),   # screened, exact ties
    dict(T=40, D=256, E=64, skew=False, adversarial=True),     # exact path, exact ties
    # screened, every expert a candidate and the winners at any list position
    dict(T=520, D=256, E=384, skew=False, clustered=True),
]


def _clustered_router(wr, seed=5):
    """Router rows all equal to row 0 except one element each, moved by 1-3 bf16 ulps:
    the logits then differ by less than the screening bound, so nearly every expert is a
    candidate and the winners sit anywhere in the candidate list."""
    wr = np.repeat(wr[:1], wr.shape[0], axis=0)
    E, D = wr.shape
    pos = np.random.default_rng(seed).integers(0, D, size=E)
    wr[np.arange(E), pos] = wr[0, pos] + (np.arange(E) % 3 + 1).astype(np.uint16)
    return wr


def _adversarial_router(h, wr):
    """Exact ties: duplicated router rows give equal logits (lower index must win), and
    all-zero hidden rows give every expert the same logit (plus bias)."""
    h, wr = h.copy(), wr.copy()
    E = wr.shape[0]
    for dst, src in [(5, 3), (E - 1, 3), (17, 40), (E // 2, 0)]:
        wr[dst] = wr[src]
    h[7] = 0
    h[-1] = 0
    h[11] = h[12]                            # two identical tokens
    return h, wr


@pytest.mark.parametrize("c", ROUTER_CASES, ids=lambda c: f"T{c['T']}_D{c['D']}_E{c['E']}_k{c.get('k', 8)}"
                         + ("_adv" if c.get("adversarial") else "") + ("_clustered" if c.get("clustered") else ""))
def test_route_bitexact(c):
    k = c.get("k", 8)
    wl = synth.custom("nvfp4", T=c["T"], D=c["D"], F=128, E=c["E"], skew=c["skew"], seed=11)
    h, wr, bias = wl.hidden(), wl.router_weight(), wl.router_bias()
    if c.get("adversarial"):
        h, wr = _adversarial_router(h, wr)
    if c.get("clustered"):
        wr = _clustered_router(wr)
    report("route", **c)
    idx, w, logits, amax = moe.route(to_dev(h), to_dev(wr), k, None if bias is None else to_dev(bias), True,
                                     want_logits=True)
    torch.cuda.synchronize()
    o_idx, o_w, o_lg = oracle.route(h, wr, k=k, bias=bias, want_logits=True)
    assert np.array_equal(host(logits).view(np.uint32), o_lg.view(np.uint32)), "logits differ"
    assert np.array_equal(host(idx), o_idx), "top-k indices differ"
    np.testing.assert_allclose(host(w), o_w, rtol=1e-6, atol=0)  # fp64 exp of two libraries
    ref_amax = np.abs(synth.bf16_to_f32(h)).max()
    assert host(amax)[0] == ref_amax
    # without the logits request the same indices and weights come out
    d_bias = None if bias is None else to_dev(bias)
    idx2, w2, _, _ = moe.route(to_dev(h), to_dev(wr), k, d_bias)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx2), o_idx) and np.array_equal(host(w2), host(w))
    if c["T"] >= 512:
        # screened batch vs the exact path on its first 256 tokens: identical bits
        idx3, w3, _, _ = moe.route(to_dev(h[:256]), to_dev(wr), k, d_bias)
        torch.cuda.synchronize()
        assert np.array_equal(host(idx3), host(idx)[:256])
        assert np.array_equal(host(w3).view(np.uint32), host(w)[:256].view(np.uint32))


# ------------------------------------------------------------------ layer
LAYER_CASES = [
    dict(name="tiny-nvfp4", wl=synth.WORKLOADS[0]),
    dict(name="decode-nvfp4", wl=synth.custom("nvfp4", T=40, D=256, F=256, E=16, seed=21)),
    dict(name="decode-mxfp8", wl=synth.custom("mxfp8", T=40, D=256, F=256, E=16, seed=22)),
    dict(name="decode-nvfp4-k384", wl=synth.custom("nvfp4", T=24, D=512, F=384, E=12, seed=23)),
    dict(name="decode-mxfp8-k384", wl=synth.custom("mxfp8", T=24, D=512, F=384, E=12, seed=24)),
    dict(name="prefill-nvfp4", wl=synth.custom("nvfp4", T=300, D=256, F=256, E=16, seed=25)),
    dict(name="prefill-mxfp8", wl=synth.custom("mxfp8", T=300, D=256, F=256, E=16, seed=26)),
    dict(name="ep-share-nvfp4", wl=synth.custom("nvfp4", T=64, D=256, F=128, E=32, e_begin=8, e_end=20, seed=27)),
    dict(name="ep-share-prefill-mxfp8",
         wl=synth.custom("mxfp8", T=400, D=256, F=128, E=24, e_begin=0, e_end=6, seed=28)),
    dict(name="skew-mxfp8", wl=synth.custom("mxfp8", T=256, D=256, F=256, E=64, skew=True, seed=29)),
    dict(name="skew-prefill-nvfp4", wl=synth.custom("nvfp4", T=600, D=256, F=128, E=16, skew=True, seed=30)),
    # prefill shapes with longer K on the 64-row MFMA tiles
    dict(name="prefill-nvfp4-k1024", wl=synth.custom("nvfp4", T=1024, D=1024, F=512, E=32, seed=37)),
    dict(name="prefill-mxfp8-k1024", wl=synth.custom("mxfp8", T=1024, D=1024, F=512, E=32, seed=38)),
    # skewed routing on the MFMA tile kernels: hot experts fill several M-tiles while cold
    # ones end in short tails (MXFP8's 128-row tiles run tails of <= 64 rows on half the
    # subtiles, longer tails on all of them)
    dict(name="prefill-mxfp8-skew-tiles", wl=synth.custom("mxfp8", T=1100, D=512, F=256, E=24, skew=True, seed=39)),
    dict(name="prefill-nvfp4-skew-tiles", wl=synth.custom("nvfp4", T=1100, D=512, F=256, E=24, skew=True, seed=40)),
    # NVFP4 prefill on the 256 x 256 tiles at widths that are not powers of two (5 gate_up
    # N-blocks, 3 down N-blocks, 12 and 10 K chunks; about 470 rows per expert: two tiles)
    dict(name="prefill-nvfp4-d768-f640", wl=synth.custom("nvfp4", T=700, D=768, F=640, E=12, seed=59)),
    # decode shapes with K a multiple of 512 run the streaming kernels
    dict(name="stream-nvfp4-k2048", wl=synth.custom("nvfp4", T=48, D=2048, F=1536, E=16, seed=31)),
    dict(name="stream-mxfp8-k2048", wl=synth.custom("mxfp8", T=48, D=2048, F=1536, E=16, seed=32)),
    dict(name="stream-mxfp8-k4096-k512", wl=synth.custom("mxfp8", T=24, D=4096, F=512, E=8, seed=33)),
    dict(name="stream-nvfp4-full-dims", wl=synth.custom("nvfp4", T=64, D=4096, F=2560, E=16, seed=34)),
    dict(name="stream-mxfp8-full-dims", wl=synth.custom("mxfp8", T=64, D=4096, F=2560, E=16, seed=35)),
    dict(name="stream-nvfp4-ep-share", wl=synth.custom("nvfp4", T=64, D=2048, F=1024, E=32, e_begin=4, e_end=12,
                                                       seed=36)),
    # OCP MXFP4 (W4A4) on the scaled FP4 MFMA: decode and prefill batches, ragged tiles,
    # several N blocks, an expert-parallel share, skewed routing and the full dimensions
    dict(name="decode-mxfp4", wl=synth.custom("mxfp4", T=40, D=256, F=256, E=16, seed=51)),
    dict(name="prefill-mxfp4", wl=synth.custom("mxfp4", T=300, D=256, F=256, E=16, seed=52)),
    dict(name="prefill-mxfp4-k1024", wl=synth.custom("mxfp4", T=1024, D=1024, F=512, E=32, seed=53)),
    dict(name="ep-share-mxfp4", wl=synth.custom("mxfp4", T=400, D=512, F=384, E=24, e_begin=6, e_end=15, seed=54)),
    dict(name="skew-mxfp4", wl=synth.custom("mxfp4", T=600, D=256, F=128, E=16, skew=True, seed=55)),
    dict(name="mxfp4-full-dims", wl=synth.custom("mxfp4", T=64, D=4096, F=2560, E=16, seed=56)),
    # the longest K whose activation row scales the MX kernel stages in LDS (8192: 64 dwords
    # per row) and a down K of 10 chunks (5 dwords per row; the last 4-chunk group half full)
    dict(name="prefill-mxfp4-k8192", wl=synth.custom("mxfp4", T=160, D=8192, F=640, E=8, seed=57)),
    # the same limit for MXFP8 at prefill (weight scales exchanged per ring turn), and a
    # down K of 3 dwords per row
    dict(name="prefill-mxfp8-k8192", wl=synth.custom("mxfp8", T=160, D=8192, F=384, E=8, seed=58)),
    # three 256-wide weight tiles and a down K of six chunks (MX: the last 4-chunk group of
    # MXFP4 half full, three MXFP8 ring turns), prefill-shaped on every scaled route
    dict(name="prefill-mxfp8-d768-f384", wl=synth.custom("mxfp8", T=500, D=768, F=384, E=10, seed=81)),
    dict(name="prefill-mxfp4-d768-f384", wl=synth.custom("mxfp4", T=500, D=768, F=384, E=10, seed=82)),
    dict(name="prefill-fp8-d768-f384", wl=synth.custom("fp8", T=500, D=768, F=384, E=10, seed=83)),
    # NVFP4 weights with bf16 activations (W4A16) on all three kernel families
    dict(name="decode-w4a16", wl=synth.custom("w4a16", T=40, D=256, F=256, E=16, seed=61)),
    dict(name="prefill-w4a16", wl=synth.custom("w4a16", T=300, D=256, F=256, E=16, seed=62)),
    dict(name="prefill-w4a16-k1024", wl=synth.custom("w4a16", T=1024, D=1024, F=512, E=32, seed=63)),
    dict(name="stream-w4a16-k2048", wl=synth.custom("w4a16", T=48, D=2048, F=1536, E=16, seed=64)),
    dict(name="stream-w4a16-full-dims", wl=synth.custom("w4a16", T=64, D=4096, F=2560, E=16, seed=65)),
    dict(name="ep-share-w4a16", wl=synth.custom("w4a16", T=400, D=512, F=384, E=24, e_begin=6, e_end=15, seed=66)),
    dict(name="skew-w4a16", wl=synth.custom("w4a16", T=600, D=256, F=128, E=16, skew=True, seed=67)),
    # degenerate and extreme cases: one token, top-1, every expert taken by every token,
    # top-2 on an expert-parallel share, and 1024 experts (the router's largest table)
    dict(name="single-token-nvfp4", wl=synth.custom("nvfp4", T=1, D=256, F=128, E=16, seed=71)),
    dict(name="top1-mxfp8", wl=synth.custom("mxfp8", T=200, D=256, F=128, E=16, k=1, seed=72)),
    dict(name="all-experts-w4a16", wl=synth.custom("w4a16", T=48, D=256, F=128, E=8, seed=73)),
    dict(name="top2-ep-share-mxfp4", wl=synth.custom("mxfp4", T=300, D=256, F=128, E=32, k=2, e_begin=3, e_end=11,
                                                     seed=74)),
    dict(name="e1024-nvfp4", wl=synth.custom("nvfp4", T=64, D=128, F=128, E=1024, seed=75)),
    # bf16 experts (unquantised weights and activations) on all three kernel families
    dict(name="decode-bf16", wl=synth.custom("bf16", T=40, D=256, F=256, E=16, seed=81)),
    dict(name="prefill-bf16", wl=synth.custom("bf16", T=300, D=256, F=256, E=16, seed=82)),
    dict(name="prefill-bf16-k1024", wl=synth.custom("bf16", T=1024, D=1024, F=512, E=32, seed=83)),
    dict(name="stream-bf16-k2048", wl=synth.custom("bf16", T=48, D=2048, F=1536, E=16, seed=84)),
    dict(name="ep-share-bf16", wl=synth.custom("bf16", T=400, D=512, F=384, E=24, e_begin=6, e_end=15, seed=85)),
    # the 256 x 256 bf16 tiles: hot experts over several 256-row tiles with short tails, and
    # widths that are not powers of two (5 gate_up N-blocks, 3 down N-blocks)
    dict(name="prefill-bf16-skew-tiles", wl=synth.custom("bf16", T=1100, D=512, F=256, E=24, skew=True, seed=88)),
    dict(name="prefill-bf16-d768-f640", wl=synth.custom("bf16", T=700, D=768, F=640, E=12, seed=89)),
    # MXFP8 with exact sums (MOE_FLAG_EXACT_SUMS): the bf16 expansion on the grouped,
    # tile and streaming kernels instead of the scaled FP8 MFMA
    dict(name="decode-mxfp8-exact", wl=synth.custom("mxfp8", T=40, D=256, F=256, E=16, seed=22), flags=1),
    dict(name="prefill-mxfp8-exact", wl=synth.custom("mxfp8", T=300, D=256, F=256, E=16, seed=26), flags=1),
    dict(name="prefill-mxfp8-k1024-exact", wl=synth.custom("mxfp8", T=1024, D=1024, F=512, E=32, seed=38), flags=1),
    dict(name="prefill-mxfp8-skew-tiles-exact",
         wl=synth.custom("mxfp8", T=1100, D=512, F=256, E=24, skew=True, seed=39), flags=1),
    dict(name="ep-share-prefill-mxfp8-exact",
         wl=synth.custom("mxfp8", T=400, D=256, F=128, E=24, e_begin=0, e_end=6, seed=28), flags=1),
    dict(name="stream-mxfp8-k2048-exact", wl=synth.custom("mxfp8", T=48, D=2048, F=1536, E=16, seed=32), flags=1),
    dict(name="stream-mxfp8-full-dims-exact", wl=synth.custom("mxfp8", T=64, D=4096, F=2560, E=16, seed=35),
         flags=1),
    # the scaled FP8 MFMA at the full dimensions (decode tiles) and at widths that are not
    # powers of two (5 gate_up N-blocks, 3 down N-blocks, 12 and 10 K chunks)
    dict(name="mxfp8-full-dims", wl=synth.custom("mxfp8", T=64, D=4096, F=2560, E=16, seed=57)),
    dict(name="prefill-mxfp8-d768-f640", wl=synth.custom("mxfp8", T=700, D=768, F=640, E=12, seed=58)),
    # FP8 (E4M3, a scale per weight channel and per activation row) on the scaled FP8 MFMA
    # with unit E8M0 scales: decode and prefill tiles, an expert-parallel share, skewed
    # routing, top-1, the full dimensions, widths that are not powers of two, and hidden
    # states with an all-zero row, a tiny row and a row with one huge outlier
    dict(name="decode-fp8", wl=synth.custom("fp8", T=40, D=256, F=256, E=16, seed=80)),
    dict(name="prefill-fp8", wl=synth.custom("fp8", T=300, D=256, F=256, E=16, seed=81)),
    dict(name="prefill-fp8-ep", wl=synth.custom("fp8", T=400, D=256, F=128, E=24, e_begin=0, e_end=6, seed=82)),
    dict(name="skew-fp8", wl=synth.custom("fp8", T=1100, D=512, F=256, E=24, skew=True, seed=83)),
    dict(name="top1-fp8", wl=synth.custom("fp8", T=200, D=256, F=128, E=16, k=1, seed=84)),
    dict(name="fp8-full-dims", wl=synth.custom("fp8", T=64, D=4096, F=2560, E=16, seed=85)),
    dict(name="prefill-fp8-d768-f640", wl=synth.custom("fp8", T=700, D=768, F=640, E=12, seed=86)),
    dict(name="fp8-edge-rows", wl=synth.custom("fp8", T=96, D=512, F=256, E=16, seed=87), edge_rows=True),
    # NVFP4 weights whose block scales are E4M3 subnormals, on the streaming (NVFP4 and
    # W4A16), prefill tile and grouped kernels
    dict(name="stream-nvfp4-subnormal-scales", wl=synth.custom("nvfp4", T=40, D=1024, F=512, E=16, seed=91),
         subnormal_w=True),
    dict(name="prefill-nvfp4-subnormal-scales", wl=synth.custom("nvfp4", T=600, D=1024, F=512, E=16, seed=92),
         subnormal_w=True),
    dict(name="stream-w4a16-subnormal-scales", wl=synth.custom("w4a16", T=40, D=1024, F=512, E=16, seed=93),
         subnormal_w=True),
    dict(name="grouped-nvfp4-subnormal-scales", wl=synth.custom("nvfp4", T=24, D=512, F=384, E=12, seed=94),
         subnormal_w=True),
]


def _edge_rows(h: np.ndarray) -> np.ndarray:
    """Hidden states with an all-zero row (row scale 1, every code 0), a row scaled by
    2^-60 (a tiny row scale) and a row whose one huge value pushes the rest of it into
    E4M3's subnormals."""
    h = h.copy()
    h[3] = 0
    h[7] = synth.normal_bf16(1, 11, 0, h.shape[1], 2.0 ** -60)
    h[11, 5] = 0x4B00  # 2^23 in bf16
    return h


def _subnormal_weight_scales(h: np.ndarray, gu: np.ndarray, dn: np.ndarray):
    """Masters whose NVFP4 block scales are E4M3 subnormals. In every expert one 16-block
    of 4096s sets the tensor scale, which puts every other block's scale below 2^-6. That
    block only ever meets zeros: it sits in hidden features 0..15, which are zeroed, and
    in the down columns of intermediate features 0..15, whose gate rows are zero (SwiGLU
    of a zero gate is zero). So every output element comes from subnormally scaled
    blocks."""
    h, gu, dn = h.copy(), gu.copy(), dn.copy()
    h[:, :16] = 0
    gu[:, :16, :] = 0
    gu[:, 16, :16] = 0x4580  # bf16 4096
    dn[:, 0, :16] = 0x4580
    return h, gu, dn


@pytest.mark.parametrize("c", LAYER_CASES, ids=lambda c: c["name"])
def test_forward_parity(c):
    wl = c["wl"]
    fmt, T, D, F, E, k = wl.fmt, wl.T, wl.D, wl.F, wl.E, wl.k
    eb, ee = wl.e_begin, wl.local_end
    h, wr, bias, gu_m, dn_m = case_inputs(wl)
    if c.get("edge_rows"):
        h = _edge_rows(h)
    if c.get("subnormal_w"):
        h, gu_m, dn_m = _subnormal_weight_scales(h, gu_m, dn_m)
    report("forward", case=c["name"], fmt=fmt, T=T, D=D, F=F, E=E, local=(eb, ee))

    # GPU: quantise, route, forward with every tap
    gu = moe.quantize_weights(fmt, to_dev(gu_m))
    dn = moe.quantize_weights(fmt, to_dev(dn_m))
    d_h = to_dev(h)
    idx, w, _, amax = moe.route(d_h, to_dev(wr), k, None if bias is None else to_dev(bias), True)
    layer = moe.Layer(fmt, T, D, F, E, gu, dn, top_k=k, e_begin=eb, e_end=ee, flags=c.get("flags", 0))
    native8 = scaled_fp8(layer)
    report("  plan", **layer.plan())
    taps = layer.enable_taps()
    out = host(layer.forward(d_h, idx, w, h_amax=amax if fmt == "nvfp4" else None))
    torch.cuda.synchronize()
    tp = {k_: host(v) for k_, v in taps.items()}

    # oracle: its own quantised weights (bf16 experts: the masters), routing and layer
    if fmt == "bf16":
        o_dn = dn_m
        wkw = dict(gate_up_master=gu_m, down_master=dn_m)
    else:
        o_gu, o_dn = oracle.quantize_weights(fmt, gu_m), oracle.quantize_weights(fmt, dn_m)
        wkw = dict(gate_up=o_gu, down=o_dn)
    o_idx, o_w = oracle.route(h, wr, k=k, bias=bias)
    assert np.array_equal(host(idx), o_idx)
    ref, otp = oracle.moe_forward(fmt, h, o_idx, o_w, D=D, F=F, E=E, e_begin=eb, e_end=ee, taps=True, **wkw)
    counts, offs, ss = oracle.permute(o_idx, eb, ee)
    S = int(offs[-1])

    # bit-exact: permutation and hidden-state quantisation
    assert np.array_equal(tp["counts"], counts)
    assert np.array_equal(tp["offsets"], offs)
    assert np.array_equal(tp["sorted_slot"][:S], ss)
    if fmt not in ("w4a16", "bf16"):  # W4A16 and bf16 experts keep the hidden states in bf16
        assert np.array_equal(tp["a_codes"], otp["a_codes"]), "hidden-state codes differ"
    if fmt == "fp8":  # the row scales
        assert np.array_equal(tp["a_tscale"].view(np.uint32), otp["a_tscale"].view(np.uint32)), "row scales differ"
    elif fmt not in ("w4a16", "bf16"):
        assert np.array_equal(tp["a_scales"], otp["a_scales"]), "hidden-state scales differ"
    if fmt == "nvfp4":
        assert tp["a_tscale"][0] == otp["a_tscale"][0]

    # intermediate: values close to the oracle's, codes exact given the GPU's own values
    g_inter = tp["inter"][:S]
    scale_i = np.abs(otp["inter"]).max()
    inter_err = float(np.abs(g_inter - otp["inter"]).max()) / scale_i
    g_its = tp["inter_tscale"][0] if fmt == "nvfp4" else None
    g_iscales = tp["inter_scales"][:S] if "inter_scales" in tp else None
    o_iscales = otp.get("inter_scales")
    if fmt == "fp8":  # fp32 row scales in place of block scales
        g_iscales, o_iscales = tp["inter_tscale"][:S], otp["inter_tscale"]
    check_intermediate_codes(fmt, g_inter, tp["inter_codes"][:S], g_iscales, g_its)
    inter_tol = INTER_TOL_SCALED_FP8 if native8 else INTER_TOL_EXACT
    assert inter_err < inter_tol, f"SwiGLU intermediate differs by {inter_err:.2e} of its max"

    # output: stage-wise on every token, independent on tokens without intermediate flips
    e_stage, e_ind, flips, excluded = check_outputs(
        fmt, out, ref, o_idx, o_w, tp["inter_codes"][:S], g_iscales, g_its, otp["inter_codes"],
        o_iscales, ss, o_dn, D=D, F=F, E=E, e_begin=eb, e_end=ee, **output_bounds(native8))
    report("  result", S=S, inter_rel=f"{inter_err:.2e}", code_flips=flips, tokens_with_flips=excluded,
           stage_err=f"{e_stage:.2e}", independent_err=f"{e_ind:.2e}")
    has_local = ((o_idx >= eb) & (o_idx < ee)).any(1)
    assert not out[~has_local].any(), "tokens without a local slot must be zero"


def test_empty_batch_is_a_no_op():
    wl = synth.WORKLOADS[0]
    gu = moe.quantize_weights("nvfp4", to_dev(wl.gate_up_master(0, wl.E)))
    dn = moe.quantize_weights("nvfp4", to_dev(wl.down_master(0, wl.E)))
    layer = moe.Layer("nvfp4", 0, wl.D, wl.F, wl.E, gu, dn)
    out = torch.empty((0, wl.D), dtype=torch.float32, device="cuda")
    empty_i = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    empty_w = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    empty_h = torch.empty((0, wl.D), dtype=torch.int16, device="cuda")
    layer.forward(empty_h, empty_i, empty_w, out=out)
    torch.cuda.synchronize()


def test_repeat_calls_are_deterministic():
    """Same inputs, same bytes: the forward reuses its workspace without stale state."""
    wl = synth.custom("nvfp4", T=40, D=256, F=256, E=16, seed=41)
    h, wr, _, gu_m, dn_m = case_inputs(wl)
    gu, dn = moe.quantize_weights("nvfp4", to_dev(gu_m)), moe.quantize_weights("nvfp4", to_dev(dn_m))
    d_h = to_dev(h)
    idx, w, _, _ = moe.route(d_h, to_dev(wr), 8)
    layer = moe.Layer("nvfp4", wl.T, wl.D, wl.F, wl.E, gu, dn)
    a = host(layer.forward(d_h, idx, w)).copy()
    b = host(layer.forward(d_h, idx, w))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "fp8", "w4a16", "bf16"])
def test_expert_parallel_shares_add_up(fmt):
    """The expert-parallel contract on the GPU: four expert ranges (an EP4 split, each one
    rank's moe_forward) sum to the whole layer's output, and every share's tokens without a
    local slot are zero. NVFP4 is excluded: its intermediate tensor scale is taken over
    each share's own slots, as the oracle's is."""
    wl = synth.custom(fmt, T=300, D=256, F=256, E=32, seed=95)
    h, wr, bias, gu_m, dn_m = case_inputs(wl)
    report("ep shares", fmt=fmt, T=wl.T, E=wl.E)
    gu, dn = moe.quantize_weights(fmt, to_dev(gu_m)), moe.quantize_weights(fmt, to_dev(dn_m))
    d_h = to_dev(h)
    idx, w, _, _ = moe.route(d_h, to_dev(wr), wl.k)
    full = host(moe.Layer(fmt, wl.T, wl.D, wl.F, wl.E, gu, dn).forward(d_h, idx, w)).astype(np.float64)
    o_idx = host(idx)
    parts = np.zeros_like(full)
    for r in range(4):
        eb, ee = 8 * r, 8 * r + 8
        part = host(moe.Layer(fmt, wl.T, wl.D, wl.F, wl.E, gu, dn, e_begin=eb, e_end=ee).forward(d_h, idx, w))
        local = ((o_idx >= eb) & (o_idx < ee)).any(1)
        assert not part[~local].any(), f"share {r}: tokens without a local slot must be zero"
        parts += part
    np.testing.assert_allclose(parts, full, rtol=0, atol=2e-6 * np.abs(full).max())


# ------------------------------------------------------------------ graph replay
GRAPH_CASES = [
    dict(name="decode-nvfp4", wl=synth.custom("nvfp4", T=64, D=256, F=256, E=16, seed=41)),     # one-workgroup permute
    dict(name="prefill-mxfp8", wl=synth.custom("mxfp8", T=1100, D=256, F=256, E=16, seed=42)),  # count/scan/scatter + fill
    dict(name="prefill-mxfp4", wl=synth.custom("mxfp4", T=700, D=256, F=256, E=16, seed=43)),
    dict(name="decode-w4a16", wl=synth.custom("w4a16", T=64, D=512, F=256, E=16, seed=44)),
    dict(name="prefill-fp8", wl=synth.custom("fp8", T=700, D=256, F=256, E=16, seed=45)),
]


@pytest.mark.parametrize("c", GRAPH_CASES, ids=lambda c: c["name"])
def test_graph_replay_matches_eager(c):
    """route + forward captured as one HIP graph: every replay equals the eager step bit for
    bit, with eager launches and synchronisations between the replays."""
    wl = c["wl"]
    h, wr, bias, gu_m, dn_m = case_inputs(wl)
    report("graph", case=c["name"], T=wl.T, D=wl.D, F=wl.F, E=wl.E)
    d_h, d_wr = to_dev(h), to_dev(wr)
    gu, dn = moe.quantize_weights(wl.fmt, to_dev(gu_m)), moe.quantize_weights(wl.fmt, to_dev(dn_m))
    layer = moe.Layer(wl.fmt, wl.T, wl.D, wl.F, wl.E, gu, dn, top_k=wl.k)
    ws = moe.route_workspace(wl.T, wl.D, wl.E)
    nv = wl.fmt == "nvfp4"
    out = torch.empty((wl.T, wl.D), dtype=torch.float32, device="cuda")

    def step(dst):
        idx, w, _, amax = moe.route(d_h, d_wr, wl.k, want_amax=nv, workspace=ws)
        layer.forward(d_h, idx, w, out=dst, h_amax=amax)

    step(out)
    torch.cuda.synchronize()
    eager = host(out).copy()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step(out)
    other = torch.empty_like(out)
    for r in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), eager.view(np.uint32)), f"replay {r} differs from eager"
        step(other)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(host(other).view(np.uint32), eager.view(np.uint32))
