"""Evidence for the NVFP4 scale handling on the GPU (CPU only, the oracle's arithmetic).

The expert GEMMs must take NVFP4 operands, E2M1 codes c with one E4M3 scale s per 16
values (vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview"; AI Primer
"Thinking Machines releases Inkling 2 Small weights under Apache 2.0", section "TL;DR"),
while the gfx950 scaled MFMA takes one E8M0 (power-of-two) scale per 32 values. Two
routes: dequantise c * s exactly to a 16-bit MFMA operand, or fold s into FP8 / FP4
operands under an E8M0 scale per 32.
 1. c * s is exact in fp16 and bf16 for every code and every finite E4M3 scale (at most 6
    significant bits, magnitudes 2^-10 .. 2688): the 16-bit route computes the specified
    products exactly.
 2. The fold is not exact: re-encoding the block-scaled values per 32 by the OCP MX rule
    (oracle.fold_to_mx) changes a large share of the weight, activation and intermediate
    values, and the layer output on the tiny configuration and on decode-nvfp4's shapes
    moves by far more than the 2e-3 x RMS bar.
"""
import numpy as np

import oracle
import synth

f32 = np.float32


def test_nvfp4_values_are_exact_in_16_bit():
    codes = np.array([oracle.e2m1_value(c) for c in range(16)])
    scales = np.array([oracle.e4m3_value(b) for b in range(0x7F)])  # every finite non-negative E4M3
    v = (codes[:, None] * scales[None, :]).ravel()                   # exact in fp64
    nz = v[v != 0]
    assert np.abs(nz).min() == 2.0 ** -10 and np.abs(nz).max() == 6 * 448
    m, _ = np.frexp(np.abs(nz))
    assert np.all(np.mod(np.ldexp(m, 6), 1.0) == 0)                  # <= 6 significant bits
    assert np.array_equal(v.astype(np.float16).astype(np.float64), v)
    bf = synth.bf16_to_f32(oracle.round_bf16(v.astype(f32))).astype(np.float64)
    assert np.array_equal(bf, v)


def _nvfp4_layer(wl, W, fold=None):
    """The NVFP4 layer composed from the oracle's quantisers on T tokens, every operand of
    the expert GEMMs (block-scaled values, tensor scales applied after the sums) passed
    through `fold` (None: exact). W: expert -> the oracle's (gate_up, down) quantisation,
    filled on first use. Returns (output [T, D], changed-value shares, routing)."""
    T, D, F, E, k = wl.T, wl.D, wl.F, wl.E, wl.k
    h, wr = wl.hidden(), wl.router_weight()
    idx, w = oracle.route(h, wr, k=k)
    ac, as_, a_ts = oracle.quant_nvfp4(synth.bf16_to_f32(h))
    A = oracle.dequant_nvfp4(ac, as_, 1.0, with_tensor=False)
    counts, offs, ss = oracle.permute(idx, 0, E)
    S = len(ss)
    used = np.nonzero(counts)[0]
    for e in used:
        if e not in W:
            W[e] = tuple(oracle.quantize_weights("nvfp4", m)
                         for m in (wl.gate_up_master(int(e)), wl.down_master(int(e))))
    changed = {}

    def op(name, x):
        if fold is None:
            return x
        y = fold(x)
        n, c = changed.get(name, (0, 0))
        changed[name] = (n + x.size, c + int(np.count_nonzero(y != x)))
        return y

    Af = op("activations", A)
    inter = np.zeros((S, F), f32)
    for el in used:
        p0, p1 = offs[el], offs[el + 1]
        gu = W[el][0]
        Wg = op("weights", oracle.dequant_nvfp4(gu["codes"][0], gu["scales"][0], 1.0, with_tensor=False))
        g = (Af[ss[p0:p1] // k] @ Wg.T).astype(f32) * f32(a_ts * gu["tensor_scale"][0])
        g = g.astype(f32)
        gate, up = g[:, :F].astype(np.float64), g[:, F:].astype(np.float64)
        inter[p0:p1] = (gate * up / (1.0 + np.exp(-gate))).astype(f32)
    ic, is_, i_ts = oracle.quant_nvfp4(inter)
    I = op("intermediate", oracle.dequant_nvfp4(ic, is_, 1.0, with_tensor=False))
    out = np.zeros((T, D))
    for el in used:
        p0, p1 = offs[el], offs[el + 1]
        dn = W[el][1]
        Wd = op("weights", oracle.dequant_nvfp4(dn["codes"][0], dn["scales"][0], 1.0, with_tensor=False))
        y = ((I[p0:p1] @ Wd.T).astype(f32) * f32(i_ts * dn["tensor_scale"][0])).astype(f32)
        for p in range(p0, p1):
            t, j = divmod(int(ss[p]), k)
            out[t] += float(w[t, j]) * y[p - p0].astype(np.float64)
    return out, {n: c / m for n, (m, c) in changed.items()}, (idx, w, h)


def _check_fold(wl, report):
    W = {}
    exact, _, (idx, w, h) = _nvfp4_layer(wl, W)
    # the composition is the oracle's own layer
    used = np.unique(idx)
    remap = np.full(wl.E, -1, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    cat = lambda j: {key: np.concatenate([W[e][j][key] for e in used]) for key in ("codes", "scales", "tensor_scale")}
    ref = oracle.moe_forward("nvfp4", h, remap[idx], w, D=wl.D, F=wl.F, E=len(used), gate_up=cat(0), down=cat(1))
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    assert float(np.abs(exact - ref).max()) <= 1e-6 * rms
    for target in ("mxfp8", "mxfp4"):
        out, share, _ = _nvfp4_layer(wl, W, fold=lambda x: oracle.fold_to_mx(x, target))
        err = float(np.abs(out - exact).max()) / rms
        rel_rms = float(np.sqrt(np.mean((out - exact) ** 2))) / rms
        report[target] = dict(share, max_err_over_rms=err, rel_rms=rel_rms)
        print(f"{wl.name} T={wl.T} fold to {target}: changed values "
              + ", ".join(f"{n} {v:.1%}" for n, v in sorted(share.items()))
              + f"; output max error {err:.2e} x RMS, RMS error {rel_rms:.2e}")
        assert err > 2e-3 and share["weights"] > 0.05 and share["activations"] > 0.05


def test_fold_on_the_tiny_configuration():
    rep = {}
    _check_fold(synth.WORKLOADS[0], rep)
    assert rep["mxfp4"]["rel_rms"] > rep["mxfp8"]["rel_rms"]


def test_fold_on_decode_nvfp4_shapes():
    """decode-nvfp4's shapes, value recipe and seed (d_model 4096, d_ff 2560, 384 experts),
    on its first 4 tokens as the batch (about 30 experts: the oracle quantises each)."""
    wl1 = synth.WORKLOADS[1]
    wl = synth.Workload(1, wl1.name, "nvfp4", T=4, D=wl1.D, F=wl1.F, E=wl1.E, seed=wl1.seed)
    _check_fold(wl, {})
