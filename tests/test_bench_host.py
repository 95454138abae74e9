"""Host-side pieces of bench.py (no GPU): the oracle baseline on small samples, including an
expert-parallel share whose first tokens reach no local expert and samples that touch fewer
experts than top_k, and the multi-GPU refusal."""
import subprocess
import sys

import bench
import synth


def test_cpu_baseline_small_samples():
    cases = [synth.WORKLOADS[0],
             synth.custom("nvfp4", T=512, D=256, F=128, E=64, e_begin=0, e_end=16, seed=5),
             synth.custom("mxfp8", T=512, D=256, F=128, E=64, skew=True, seed=6),
             synth.custom("bf16", T=64, D=256, F=128, E=64, e_begin=0, e_end=8, seed=7),
             synth.custom("fp8", T=64, D=256, F=128, E=64, seed=8)]
    for wl in cases:
        r = bench.cpu_baseline(wl, wl.hidden(), wl.router_weight(), wl.router_bias(), target_s=0.2)
        assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1 and r["cpu_model"]


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stderr
