"""moe_forward_static (the entry point that allocates nothing: its workspace is the library's
static device array) against moe_forward on the same inputs, through the C ABI: the same
kernels and plan, so the outputs must be identical bit for bit. Two calls in a row, the
second with fewer tokens, so stale contents of the shared array from the first call would
show; the NVFP4 decode, MXFP8 decode (scaled FP8 MFMA) and NVFP4 grouped-kernel shapes."""
import numpy as np
import pytest
import torch

import block_scaled_moe_amd as moe
import synth
from gpu_util import case_inputs, host, report, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    dict(name="stream-nvfp4", fmt="nvfp4", T=(64, 24), D=2048, F=1536, E=16, seed=91),
    dict(name="scaled-mxfp8", fmt="mxfp8", T=(256, 40), D=1024, F=512, E=32, seed=92),
    dict(name="grouped-nvfp4", fmt="nvfp4", T=(40, 7), D=256, F=256, E=16, seed=93),
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: c["name"])
def test_forward_static_matches_forward(c):
    T0 = c["T"][0]
    wl = synth.custom(c["fmt"], T=T0, D=c["D"], F=c["F"], E=c["E"], seed=c["seed"])
    h, wr, _, gu_m, dn_m = case_inputs(wl)
    gu, dn = moe.quantize_weights(wl.fmt, to_dev(gu_m)), moe.quantize_weights(wl.fmt, to_dev(dn_m))
    nv = wl.fmt == "nvfp4"
    for T in c["T"]:
        d_h = to_dev(h[:T])
        idx, w, _, amax = moe.route(d_h, to_dev(wr), wl.k, want_amax=nv)
        layer = moe.Layer(wl.fmt, T, wl.D, wl.F, wl.E, gu, dn, top_k=wl.k)
        assert layer.workspace_bytes <= moe.STATIC_SCRATCH_BYTES
        ref = torch.full((T, wl.D), float("nan"), dtype=torch.float32, device="cuda")
        got = torch.full((T, wl.D), float("nan"), dtype=torch.float32, device="cuda")
        layer.forward_static(d_h, idx, w, out=got, h_amax=amax)
        layer.forward(d_h, idx, w, out=ref, h_amax=amax)
        torch.cuda.synchronize()
        r, g = host(ref), host(got)
        report("forward_static", case=c["name"], T=T, plan=layer.plan()["gate_up_kernel"])
        assert np.isfinite(r).all()
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"T={T}: moe_forward_static differs"
