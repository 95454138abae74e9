"""Helpers shared by the GPU parity tests: device transfer of the seeded inputs and
the oracle side of each comparison. Inputs come from synth (host), expected values
from oracle/ only."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) or other numpy arrays -> device tensor (same bytes)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rms(x: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.asarray(x, np.float64) ** 2)))


def report(name: str, **kv):
    print(name + ": " + ", ".join(f"{k}={v}" for k, v in kv.items()), flush=True)


def case_inputs(wl: synth.Workload):
    """Host inputs of a small workload: hidden, router weight, bias and all expert masters."""
    return (wl.hidden(), wl.router_weight(), wl.router_bias(), wl.gate_up_master(0, wl.E),
            wl.down_master(0, wl.E))


def check_intermediate_codes(fmt: str, inter: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                             tscale: float | None):
    """The GPU's intermediate codes equal the oracle quantiser applied to the GPU's own
    pre-quantisation fp32 values (bit-exact), for the S computed rows."""
    if fmt == "nvfp4":
        oc, os_, ots = oracle.quant_nvfp4(inter)
        assert np.float32(tscale) == ots, f"intermediate tensor scale {tscale} != {ots}"
    else:
        oc, os_ = oracle.quant_mxfp8(inter)
    bad_c = int(np.count_nonzero(oc != codes))
    bad_s = int(np.count_nonzero(os_ != scales))
    assert bad_c == 0 and bad_s == 0, f"intermediate codes differ: {bad_c} code bytes, {bad_s} scale bytes"
