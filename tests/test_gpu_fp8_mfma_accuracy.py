"""Characterisation of the gfx950 MFMA routes for MXFP8 dot products (OCP MX: E4M3 codes
with one E8M0 scale per 32 values, the format of the layers 40-47 experts in the vLLM
recipe "thinkingmachines/Inkling-2-Small", section "Overview").

tests/probe/fp8_mfma_probe.hip computes 32 x 32 tiles of dot products over K on the GPU
by (a) the scaled FP8 MFMA v_mfma_scale_f32_32x32x64_f8f6f4 on the codes and scales as
stored, chained through the MFMA accumulator for `group` 64-wide K chunks at a time and
summed in fp32 between groups, and (b) the exact bf16 expansion on the bf16 MFMA. The
exact dot products come from the oracle's dequantised operands in fp64 (each product is
exact in fp64; the fp64 sum of at most 4096 terms is within 5e-13 of the sum of
|products|). Errors are reported relative to the sum of |products|, the scale that
bounds any fp32 summation order.

What it establishes (asserted below):
 - operand layout of the 8-bit scaled MFMA: a lane's registers 0-3 hold 16 values of the
   chunk's first 32-block and registers 4-7 16 values of the second, and the scale byte
   of lane l belongs to block l / 32 of row l % 32. Layout 1 (k = 16g..+15, 32+16g..+15
   for lane half g) and layout 2 (four 8-byte pieces) agree and are exact up to the
   instruction's rounding; layout 0 (a lane's 32 contiguous k) scales half of each
   lane's values by the wrong block and is off by percents;
 - the scaled FP8 MFMA's error lies inside the instruction: restarting its accumulator
   from zero every chunk (or every 4) and summing in fp32 gives the same error as
   chaining all of K, about 2e-6 of the sum of |products| on the layer's values, 100x
   the bf16 route's 2e-8; with widely spread block scales it grows to about 2.4e-5.

Inputs: MXFP8 codes of bf16 N(0, 1) activations and N(0, 0.02) weights (the layer's
value recipe), and the same with each 32-block multiplied by 2^j, j uniform in
[-12, 12], so that block scales spread widely.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import report

pytestmark = pytest.mark.gpu

_PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libfp8probe.so")
TILES = 16


def _lib():
    if not os.path.exists(_PROBE):
        pytest.fail(f"{_PROBE} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_PROBE)
    lib.fp8_probe.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 5
    lib.fp8_probe.restype = ctypes.c_int
    return lib


def _operand(seed, stream, rows, K, sigma, spread, rng):
    x = synth.bf16_to_f32(synth.normal_bf16(seed, stream, 0, rows * K, sigma)).reshape(rows, K)
    if spread:
        x = x * np.exp2(rng.integers(-12, 13, size=(rows, K // 32))).repeat(32, axis=1).astype(np.float32)
    codes, scales = oracle.quant_mxfp8(x)
    assert scales.min() >= 1, "the probe's bf16 route needs scale codes >= 1"
    return codes, scales, oracle.dequant_mxfp8(codes, scales)


def _run(lib, mode, group, layout, K, ac, as_, bc, bs):
    dev = torch.device("cuda")
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (ac, as_, bc, bs)]
    out = torch.empty((TILES, 32, 32), dtype=torch.float32, device=dev)
    rc = lib.fp8_probe(mode, group, layout, K, TILES, *[x.data_ptr() for x in t], out.data_ptr())
    assert rc == 0, f"fp8_probe returned {rc}"
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("K", [4096, 2560])
@pytest.mark.parametrize("spread", [False, True], ids=["layer-values", "spread-scales"])
def test_fp8_mfma_accuracy(K, spread):
    lib = _lib()
    rng = np.random.default_rng(1000 + K + spread)
    rows = TILES * 32
    ac, as_, A = _operand(31, 1, rows, K, 1.0, spread, rng)
    bc, bs, B = _operand(31, 2, rows, K, 0.02, spread, rng)
    A3, B3 = A.reshape(TILES, 32, K), B.reshape(TILES, 32, K)
    ref = np.einsum("tmk,tnk->tmn", A3, B3)
    mag = np.einsum("tmk,tnk->tmn", np.abs(A3), np.abs(B3))
    ok = mag > 0
    results = {}
    n_chunks = K // 64
    for name, mode, group, layout in (("bf16-expanded", 1, 1, 0), ("fp8-L0-chained", 0, n_chunks, 0),
                                      ("fp8-L1-chained", 0, n_chunks, 1), ("fp8-L2-chained", 0, n_chunks, 2),
                                      ("fp8-L1-group4", 0, 4, 1), ("fp8-L1-group1", 0, 1, 1)):
        got = _run(lib, mode, group, layout, K, ac, as_, bc, bs)
        err = got - ref
        rel = np.abs(err[ok]) / mag[ok]
        results[name] = rel.max()
        report(f"fp8 mfma K={K} {'spread' if spread else 'layer'} {name}",
               max_rel=f"{rel.max():.2e}", mean_rel=f"{rel.mean():.2e}",
               bias=f"{(err[ok] / mag[ok]).mean():+.2e}",
               fl32_exact=f"{np.mean(got == ref.astype(np.float32)):.3f}")
    if not spread:
        # the bf16 route: an fp32 chain of exact products
        assert results["bf16-expanded"] < 5e-8
        assert results["fp8-L1-chained"] < 5e-6
    else:
        assert results["bf16-expanded"] < 2e-6
        assert results["fp8-L1-chained"] < 1e-4
        assert results["fp8-L0-chained"] > 1e-2  # the wrong block association shows
    # layouts 1 and 2 put the same k in the same block: same result up to summation order
    assert abs(results["fp8-L2-chained"] - results["fp8-L1-chained"]) <= 0.05 * results["fp8-L1-chained"]
    # no gain from summing the per-chunk results in fp32: the error is inside the instruction
    for g in ("fp8-L1-group4", "fp8-L1-group1"):
        assert results[g] >= 0.5 * results["fp8-L1-chained"]
    assert results["fp8-L1-chained"] > 20 * results["bf16-expanded"]

