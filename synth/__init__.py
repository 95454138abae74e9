"""Seeded synthetic inputs for the routed-expert MoE layer.

This module draws random numbers and describes the five workloads; it holds
none of the layer's arithmetic. The CPU oracle (tests) and the HIP path (tests,
bench) both consume exactly the bytes produced here.

Value recipe (every value is a draw from the exact distribution of
bf16_RNE(sigma * Z), Z ~ N(0, 1); see synth.c):
  hidden states   N(0, 1)                  stream 1, index t*D + d
  router weight   N(0, 1/sqrt(d_model))    stream 2, index e*D + d     ([E, D])
  gate_up master  N(0, 0.02)               stream 3, index (e*2F + n)*D + d  ([E, 2F, D])
  down master     N(0, 0.02)               stream 4, index (e*D + n)*F + f   ([E, D, F])
  router bias     -1.1 * ln(rank_e), rank = 1 + seeded permutation (stream 5);
                  skewed-routing workload only
Seed of workload i is i. The second argument of N(.,.) is a standard deviation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_HIP_LIB_PATH = os.path.join(_HERE, "libsynth_hip.so")
_lib = None
_hip_lib = None
_tables: dict = {}
_dev_tables: dict = {}

STREAM_HIDDEN, STREAM_ROUTER, STREAM_GATE_UP, STREAM_DOWN, STREAM_BIAS = 1, 2, 3, 4, 5

HIPCC_FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(hip: bool = True) -> None:
    """Compile libsynth.so (gcc, plain C + OpenMP) and, if asked, libsynth_hip.so (hipcc)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    if hip:
        cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, os.path.join(_HERE, "synth_hip.hip"),
               "-o", _HIP_LIB_PATH + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(_HIP_LIB_PATH + ".tmp", _HIP_LIB_PATH)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(hip=False)
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i32, dbl, p = ctypes.c_uint64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.synth_key.argtypes = [u64, u64]
    lib.synth_key.restype = u64
    lib.synth_u64.argtypes = [u64, u64, u64]
    lib.synth_u64.restype = u64
    lib.synth_table_size.argtypes = [dbl]
    lib.synth_table_size.restype = i32
    lib.synth_build_table.argtypes = [dbl, i32, p, p]
    lib.synth_build_table.restype = None
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, p, p, p]
    lib.synth_normal_bf16.restype = None
    lib.synth_permutation.argtypes = [u64, u64, i32, p]
    lib.synth_permutation.restype = None
    lib.synth_rank_bias.argtypes = [u64, u64, i32, dbl, p]
    lib.synth_rank_bias.restype = ctypes.c_int
    _lib = lib
    return lib


def _load_hip():
    global _hip_lib
    if _hip_lib is not None:
        return _hip_lib
    if not os.path.exists(_HIP_LIB_PATH):
        raise RuntimeError(f"{_HIP_LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(_HIP_LIB_PATH)
    u64, p = ctypes.c_uint64, ctypes.c_void_p
    lib.synth_hip_normal_bf16.argtypes = [u64, u64, u64, p, p, p, p]
    lib.synth_hip_normal_bf16.restype = ctypes.c_int
    _hip_lib = lib
    return lib


def table(sigma: float):
    """(thresholds uint64[n], guide uint32[2^16]) of the bf16 sampler for sigma."""
    sigma = float(sigma)
    if sigma not in _tables:
        lib = _load()
        n = lib.synth_table_size(sigma)
        thr = np.empty(n, dtype=np.uint64)
        guide = np.empty(1 << 16, dtype=np.uint32)
        lib.synth_build_table(sigma, n, thr.ctypes.data, guide.ctypes.data)
        _tables[sigma] = (thr, guide)
    return _tables[sigma]


def key(seed: int, stream: int) -> int:
    return int(_load().synth_key(seed, stream))


def u64(seed: int, stream: int, n: int) -> int:
    return int(_load().synth_u64(seed, stream, n))


def normal_bf16(seed: int, stream: int, offset: int, count: int, sigma: float,
                out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of deviates offset..offset+count-1 of bf16(sigma*N(0,1))."""
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == count
    thr, guide = table(sigma)
    _load().synth_normal_bf16(seed, stream, offset, count, thr.ctypes.data, guide.ctypes.data,
                              out.ctypes.data)
    return out


def normal_bf16_device(seed: int, stream: int, offset: int, count: int, sigma: float, out):
    """Same bytes as normal_bf16, drawn on the GPU into a contiguous torch tensor `out`
    (int16/uint16/bfloat16, count elements) on the current stream."""
    import torch
    assert out.is_cuda and out.is_contiguous() and out.numel() == count and out.element_size() == 2
    dev = out.device.index if out.device.index is not None else torch.cuda.current_device()
    tkey = (float(sigma), dev)
    if tkey not in _dev_tables:
        thr, guide = table(sigma)
        _dev_tables[tkey] = (torch.from_numpy(thr.view(np.int64)).to(out.device),
                             torch.from_numpy(guide.view(np.int32)).to(out.device))
    dthr, dguide = _dev_tables[tkey]
    rc = _load_hip().synth_hip_normal_bf16(key(seed, stream), offset, count, dthr.data_ptr(),
                                           dguide.data_ptr(), out.data_ptr(),
                                           torch.cuda.current_stream(out.device).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_hip_normal_bf16 failed ({rc})")
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_permutation(seed, stream, n, out.ctypes.data)
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (x.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic MoE-layer workload (shapes, formats, value recipe)."""
    index: int
    name: str
    fmt: str            # "nvfp4", "mxfp8", "mxfp4", "w4a16", "bf16" or "fp8"
    T: int              # tokens
    D: int              # d_model
    F: int              # d_ff
    E: int              # routed experts
    k: int = 8          # experts per token
    e_begin: int = 0    # local expert range [e_begin, e_end) computed on this GPU
    e_end: int = -1
    skew: bool = False  # add the -1.1*ln(rank) router bias
    seed: int = 0
    w_sigma: float = 0.02
    bias_slope: float = 1.1

    @property
    def local_end(self) -> int:
        return self.E if self.e_end < 0 else self.e_end

    @property
    def router_sigma(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def hidden(self) -> np.ndarray:
        return normal_bf16(self.seed, STREAM_HIDDEN, 0, self.T * self.D, 1.0).reshape(self.T, self.D)

    def router_weight(self) -> np.ndarray:
        return normal_bf16(self.seed, STREAM_ROUTER, 0, self.E * self.D,
                           self.router_sigma).reshape(self.E, self.D)

    def router_bias(self) -> np.ndarray | None:
        if not self.skew:
            return None
        out = np.empty(self.E, dtype=np.float32)
        if _load().synth_rank_bias(self.seed, STREAM_BIAS, self.E, self.bias_slope,
                                   out.ctypes.data) != 0:
            raise ValueError("router bias needs 1 <= E <= 4096")
        return out

    def gate_up_master(self, e0: int, e1: int | None = None) -> np.ndarray:
        """bf16 [n, 2F, D] masters of experts e0..e1-1 (rows [0,F) gate, [F,2F) up)."""
        e1 = e0 + 1 if e1 is None else e1
        per = 2 * self.F * self.D
        out = normal_bf16(self.seed, STREAM_GATE_UP, e0 * per, (e1 - e0) * per, self.w_sigma)
        return out.reshape(e1 - e0, 2 * self.F, self.D)

    def gate_up_master_device(self, e0: int, e1: int, out):
        """gate_up masters of experts e0..e1-1 drawn on the GPU into `out` ([n, 2F, D], 2-byte)."""
        per = 2 * self.F * self.D
        return normal_bf16_device(self.seed, STREAM_GATE_UP, e0 * per, (e1 - e0) * per,
                                  self.w_sigma, out)

    def down_master_device(self, e0: int, e1: int, out):
        """down masters of experts e0..e1-1 drawn on the GPU into `out` ([n, D, F], 2-byte)."""
        per = self.D * self.F
        return normal_bf16_device(self.seed, STREAM_DOWN, e0 * per, (e1 - e0) * per,
                                  self.w_sigma, out)

    def down_master(self, e0: int, e1: int | None = None) -> np.ndarray:
        """bf16 [n, D, F] masters of experts e0..e1-1."""
        e1 = e0 + 1 if e1 is None else e1
        per = self.D * self.F
        out = normal_bf16(self.seed, STREAM_DOWN, e0 * per, (e1 - e0) * per, self.w_sigma)
        return out.reshape(e1 - e0, self.D, self.F)


WORKLOADS = [
    Workload(0, "tiny-nvfp4", "nvfp4", T=16, D=256, F=128, E=64, seed=0),
    Workload(1, "decode-nvfp4", "nvfp4", T=64, D=4096, F=2560, E=384, seed=1),
    Workload(2, "decode-mxfp8", "mxfp8", T=256, D=4096, F=2560, E=384, seed=2),
    Workload(3, "prefill-nvfp4-ep4", "nvfp4", T=8192, D=4096, F=2560, E=384,
             e_begin=0, e_end=96, seed=3),
    Workload(4, "skewed-mxfp8", "mxfp8", T=16384, D=4096, F=2560, E=384, skew=True, seed=4),
    # the OCP MXFP4 (W4A4) variant at the decode and expert-parallel prefill shapes
    Workload(5, "decode-mxfp4", "mxfp4", T=64, D=4096, F=2560, E=384, seed=5),
    Workload(6, "prefill-mxfp4-ep4", "mxfp4", T=8192, D=4096, F=2560, E=384,
             e_begin=0, e_end=96, seed=6),
    # NVFP4 weights with bf16 activations (W4A16) at the same two shapes
    Workload(7, "decode-w4a16", "w4a16", T=64, D=4096, F=2560, E=384, seed=7),
    Workload(8, "prefill-w4a16-ep4", "w4a16", T=8192, D=4096, F=2560, E=384,
             e_begin=0, e_end=96, seed=8),
    # bf16 experts (unquantised) at the same two shapes
    Workload(9, "decode-bf16", "bf16", T=64, D=4096, F=2560, E=384, seed=9),
    Workload(10, "prefill-bf16-ep4", "bf16", T=8192, D=4096, F=2560, E=384,
             e_begin=0, e_end=96, seed=10),
    # FP8 experts (E4M3, a scale per weight channel and per activation row) at the same shapes
    Workload(11, "decode-fp8", "fp8", T=64, D=4096, F=2560, E=384, seed=11),
    Workload(12, "prefill-fp8-ep4", "fp8", T=8192, D=4096, F=2560, E=384,
             e_begin=0, e_end=96, seed=12),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def custom(fmt: str, T: int, D: int, F: int, E: int, k: int = 8, e_begin: int = 0,
           e_end: int = -1, skew: bool = False, seed: int = 100, name: str = "custom") -> Workload:
    """A workload with the same value recipe at other sizes (parity cases)."""
    return Workload(-1, name, fmt, T=T, D=D, F=F, E=E, k=k, e_begin=e_begin, e_end=e_end,
                    skew=skew, seed=seed)
