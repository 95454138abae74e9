"""Oracle element/scale formats pinned against library routines, fixtures and closed forms."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def test_e2m1_values_match_ocp_table():
    rows = [r.split() for r in _rows("e2m1_values.txt")]
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1_value(int(code, 16))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        got = oracle.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), c
    # closed forms of the format: largest finite, smallest normal, smallest subnormal
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert sum(math.isnan(oracle.e4m3_value(c)) for c in range(256)) == 2


def test_e8m0_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()
    for c in range(255):
        assert oracle.e8m0_value(c) == ref[c] == 2.0 ** (c - 127), c
    assert math.isnan(oracle.e8m0_value(255))


def test_encode_decode_identity_on_every_finite_code():
    for c in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_value(c)) == c
    for c in range(256):
        v = oracle.e4m3_value(c)
        if not math.isnan(v):
            assert oracle.e4m3_encode(v) == c, hex(c)


def test_e2m1_midpoints_and_saturation():
    for r in _rows("e2m1_midpoints.txt"):
        v, code = r.split()
        assert oracle.e2m1_encode(float(v)) == int(code, 16), r


def test_e2m1_encode_brute_force_exact():
    """Nearest E2M1 value by exact rational distance, ties to the even code."""
    vals = [Fraction(oracle.e2m1_value(c)) for c in range(8)]
    rng = np.random.default_rng(7)
    xs = list(rng.uniform(-8, 8, 4000).astype(np.float32)) + [np.float32(m / 4) for m in range(-30, 31)]
    for x in xs:
        a = Fraction(float(abs(x)))
        if a >= vals[-1]:
            want = 7
        else:
            d = [abs(a - v) for v in vals]
            best = min(d)
            cands = [c for c in range(8) if d[c] == best]
            want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        if math.copysign(1.0, float(x)) < 0:
            want |= 8
        assert oracle.e2m1_encode(float(x)) == want, x


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    mags = np.concatenate([
        rng.uniform(0, 464, 20000),
        np.exp2(rng.uniform(-14, 8.85, 20000)),
    ]).astype(np.float32)
    # every midpoint between adjacent finite values (ties) and the values themselves
    pos = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    xs = np.concatenate([mags, -mags, mids, -mids, pos.astype(np.float32)])
    xs = xs[np.abs(xs) < 464]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(x)) for x in xs], dtype=np.uint8)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(float(xs[i]), hex(ref[i]), hex(got[i])) for i in bad[:5]]


def test_e4m3_encode_saturates_finite():
    for v in (448.0, 463.99, 464.0, 480.0, 1e6, float(np.finfo(np.float32).max)):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    # underflow: below half the smallest subnormal -> 0; the tie at 2^-10 goes to even (0)
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00
    assert oracle.e4m3_encode(2.0 ** -10 * 1.0001) == 0x01
    assert oracle.e4m3_encode(-0.0) == 0x80


def test_e8m0_scale_rule_closed_form():
    rng = np.random.default_rng(3)
    amax = np.concatenate([np.exp2(rng.uniform(-140, 120, 5000)), [1.0, 2.0, 0.5, 255.0, 256.0, 511.0]])
    for a in amax.astype(np.float32):
        if a == 0:
            continue
        m, ex = math.frexp(float(a))
        se = min(max(ex - 1 - 8, -127), 127)
        assert oracle.e8m0_code_for_amax(float(a)) == se + 127, a
    assert oracle.e8m0_code_for_amax(0.0) == 0
    # subnormal fp32 amax uses the leading-bit position
    assert oracle.e8m0_code_for_amax(float(np.float32(2.0 ** -140))) == 0  # -148 clamps to -127


def test_nvfp4_tensor_scale():
    assert oracle.nvfp4_tensor_scale(2688.0) == 1.0
    assert oracle.nvfp4_tensor_scale(0.0) == 1.0
    a = np.float32(0.1103515625)
    assert oracle.nvfp4_tensor_scale(float(a)) == float(np.float32(a) / np.float32(2688.0))


def test_bf16_rounding_matches_torch():
    """fp32 -> bf16 (nearest, ties to even), the W4A16 intermediate's rounding, against
    torch's CPU conversion: random values over the whole exponent range, exact ties of
    both parities, values one ulp either side of a tie, subnormals and signed zeros."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 0x7F800000, 200_000, dtype=np.uint32)  # finite, non-negative
    x = bits.view(np.float32)
    kept = (bits >> 16).astype(np.uint32)
    ties = ((kept << 16) | 0x8000).view(np.float32)                # exactly half an ulp
    near = np.concatenate([((kept << 16) | 0x7FFF).view(np.float32), ((kept << 16) | 0x8001).view(np.float32)])
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, 1.0, -1.0, 3.0e38, -3.0e38], np.float32)
    allx = np.concatenate([x, -x, ties, -ties, near, special]).astype(np.float32)
    got = oracle.round_bf16(allx)
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
