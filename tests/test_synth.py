"""The seeded input generator: determinism, slicing, distribution, workload recipe."""
import numpy as np
import scipy.stats

import synth


def test_counter_based_slices_agree():
    full = synth.normal_bf16(1, 3, 0, 10_000, 0.02)
    part = synth.normal_bf16(1, 3, 1234, 777, 0.02)
    assert np.array_equal(full[1234:1234 + 777], part)
    assert not np.array_equal(synth.normal_bf16(2, 3, 0, 100, 0.02), full[:100])
    assert not np.array_equal(synth.normal_bf16(1, 4, 0, 100, 0.02), full[:100])


def test_threshold_table_is_monotone_and_covers_range():
    for sigma in (1.0, 1 / 64, 0.02):
        thr, guide = synth.table(sigma)
        assert np.all(np.diff(thr.astype(np.float64)) >= 0)
        assert thr[-1] == 1 << 63
        vmax = float(synth.bf16_to_f32(np.array([len(thr) - 1], np.uint16))[0])
        assert vmax >= 10 * sigma


def test_draws_follow_the_rounded_normal():
    x = synth.bf16_to_f32(synth.normal_bf16(0, 1, 0, 2_000_000, 1.0)).astype(np.float64)
    assert abs(x.mean()) < 3e-3 and abs(x.std() - 1) < 3e-3
    ks = scipy.stats.kstest(x[:100_000] + np.random.default_rng(0).uniform(-1e-3, 1e-3, 100_000), "norm")
    assert ks.pvalue > 1e-3
    # exact probability of one bf16 value: P(bf16(Z) == 1.0) = Phi(1 + 2^-8) - Phi(1 - 2^-9)
    p = scipy.stats.norm.cdf(1 + 2 ** -8) - scipy.stats.norm.cdf(1 - 2 ** -9)
    n = np.count_nonzero(x == 1.0)
    assert abs(n - p * x.size) < 5 * np.sqrt(p * x.size)


def test_workload_shapes_and_sigmas():
    wl = synth.WORKLOADS[0]
    assert (wl.T, wl.D, wl.F, wl.E, wl.k) == (16, 256, 128, 64, 8)
    assert wl.router_sigma == 1 / 16
    wr = synth.bf16_to_f32(wl.router_weight())
    assert abs(wr.std() - 1 / 16) < 0.01
    g = synth.bf16_to_f32(wl.gate_up_master(3, 5))
    assert g.shape == (2, 256, 256) and abs(g.std() - 0.02) < 0.002
    assert np.array_equal(wl.gate_up_master(4), wl.gate_up_master(3, 5)[1:])
    assert synth.WORKLOADS[3].local_end == 96 and synth.WORKLOADS[1].local_end == 384
    b = synth.WORKLOADS[4].router_bias()
    assert b.max() == 0.0 and np.isclose(b.min(), -1.1 * np.log(384), rtol=1e-6)
    assert len(set(np.round(b, 6))) == 384
