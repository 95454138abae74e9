"""MI355X-native block-scaled routed-expert MoE layer.

A thin ctypes binding over libmoe.so (HIP kernels for gfx950 behind the C ABI of
include/moe.h). It only marshals arguments: torch provides device memory and the
current stream, and every step of the layer runs in the library's kernels. The
binding refuses to run without the built library; there is no fallback path.

The layer (vLLM recipe "thinkingmachines/Inkling-2-Small", section "Overview"; AI
Primer "Thinking Machines releases Inkling 2 Small weights under Apache 2.0",
sections "TL;DR" and "NVFP4 and MXFP8 experts"): top-8 of 384 routed experts, no
shared expert, NVFP4 or MXFP8 experts with activations quantised to the same format.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

FMT = {"nvfp4": 1, "mxfp8": 2, "mxfp4": 3, "w4a16": 4, "bf16": 5, "fp8": 6}  # w4a16: moe_forward only (NVFP4 weights)
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape", -3: "alignment",
          -4: "workspace", -5: "HIP launch failed"}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what}: status {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


class MoePacked(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class MoeRowMajor(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class MoeTaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "counts", "offsets", "sorted_slot", "a_codes", "a_scales", "a_tscale", "inter",
        "inter_codes", "inter_scales", "inter_tscale", "y")]


class MoeForwardArgs(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
                ("F", ctypes.c_int32), ("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("e_begin", ctypes.c_int32), ("e_end", ctypes.c_int32),
                ("h", ctypes.c_void_p), ("h_amax", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("gate_up", MoePacked), ("down", MoePacked), ("out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("taps", ctypes.POINTER(MoeTaps)), ("events", ctypes.c_void_p), ("flags", ctypes.c_uint32)]


class MoePlanInfo(ctypes.Structure):
    _fields_ = [("gate_up_kernel", ctypes.c_char_p), ("down_kernel", ctypes.c_char_p),
                ("m_tile_rows", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


N_EVENTS = 6  # MOE_EV_BEGIN, GATE_UP, GATE_UP_END, DOWN, DOWN_END, END
FLAG_EXACT_SUMS = 1  # MXFP8: exact bf16 expansion on the bf16 MFMA instead of the scaled FP8 MFMA


# every symbol include/moe.h declares, with its ctypes signature
SIGNATURES = {
    "moe_abi_version": ([], ctypes.c_int32),
    "moe_status_string": ([ctypes.c_int32], ctypes.c_char_p),
    "moe_quantize_weights": ([ctypes.c_void_p, ctypes.POINTER(MoePacked), ctypes.c_void_p], ctypes.c_int32),
    "moe_pack_weights": ([ctypes.POINTER(MoeRowMajor), ctypes.POINTER(MoePacked), ctypes.c_void_p], ctypes.c_int32),
    "moe_route_workspace_bytes": ([ctypes.c_int32] * 3, ctypes.c_size_t),
    "moe_route": ([ctypes.c_int32] * 4 + [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int32),
    "moe_forward_validate": ([ctypes.POINTER(MoeForwardArgs)], ctypes.c_int32),
    "moe_forward_workspace_bytes": ([ctypes.POINTER(MoeForwardArgs)], ctypes.c_size_t),
    "moe_forward": ([ctypes.POINTER(MoeForwardArgs), ctypes.c_void_p], ctypes.c_int32),
    "moe_forward_plan": ([ctypes.POINTER(MoeForwardArgs), ctypes.POINTER(MoePlanInfo)], ctypes.c_int32),
    "moe_forward_static": ([ctypes.POINTER(MoeForwardArgs), ctypes.c_void_p], ctypes.c_int32),
}
STATIC_SCRATCH_BYTES = 64 << 20  # MOE_STATIC_SCRATCH_BYTES: moe_forward_static's device array


def lib():
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise MoeError(what, rc)


@dataclasses.dataclass
class PackedWeights:
    """Device tensors of one packed matrix kind for E experts (logically [E][N][K]) in the
    tiled layout of include/moe.h: NVFP4 codes [E][N/32][K/64][32][32], MXFP8 codes
    [E][N/32][K/64][4][32][16] (the four 16-column quarters of a block apart), scales
    [E][N/32][K/64][32][4 | 2] (NVFP4 | MXFP8); MXFP4 keeps the two 32-column halves of
    a block apart, codes [E][N/32][K/64][2][32][16] and scales [E][N/32][K/64][2][32][1];
    bf16 codes [E][N/32][K/64][2][32][64]; FP8 codes as MXFP8's, no block scales and the
    channel scales in tensor_scale [E][N]."""
    fmt: str
    E: int
    N: int
    K: int
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor | None

    @staticmethod
    def empty(fmt: str, E: int, N: int, K: int, device="cuda") -> "PackedWeights":
        if fmt == "w4a16":  # a W4A16 layer's weights are NVFP4
            fmt = "nvfp4"
        if fmt not in FMT or fmt == "w4a16":
            raise ValueError(f"unknown format {fmt!r}")
        nv, f8 = fmt == "nvfp4", fmt == "fp8"
        if N % 32 or K % 64:
            raise ValueError(f"packed weights need N % 32 == 0 and K % 64 == 0 (got N={N}, K={K})")
        if fmt == "bf16":  # bf16 values in the tile layout, no scales
            codes = torch.empty((E, N // 32, K // 64, 2, 32, 64), dtype=torch.uint8, device=device)
            scales = torch.empty((0,), dtype=torch.uint8, device=device)
        elif fmt == "mxfp4":
            codes = torch.empty((E, N // 32, K // 64, 2, 32, 16), dtype=torch.uint8, device=device)
            scales = torch.empty((E, N // 32, K // 64, 2, 32, 1), dtype=torch.uint8, device=device)
        elif f8:  # E4M3 codes in MXFP8's order; one fp32 scale per output channel
            codes = torch.empty((E, N // 32, K // 64, 4, 32, 16), dtype=torch.uint8, device=device)
            scales = torch.empty((E, 0), dtype=torch.uint8, device=device)
        else:
            codes = torch.empty((E, N // 32, K // 64, 4, 32, 16) if fmt == "mxfp8" else (E, N // 32, K // 64, 32, 32),
                                dtype=torch.uint8,
                                device=device)
            scales = torch.empty((E, N // 32, K // 64, 32, 4 if nv else 2), dtype=torch.uint8, device=device)
        ts = (torch.empty(E, dtype=torch.float32, device=device) if nv else
              torch.empty((E, N), dtype=torch.float32, device=device) if f8 else None)
        return PackedWeights(fmt, E, N, K, codes, scales, ts)

    def experts(self, e0: int, e1: int) -> "PackedWeights":
        """View of experts e0..e1-1 (contiguous slices of the same buffers)."""
        return PackedWeights(self.fmt, e1 - e0, self.N, self.K, self.codes[e0:e1], self.scales[e0:e1],
                             None if self.tensor_scale is None else self.tensor_scale[e0:e1])

    def struct(self) -> MoePacked:
        return MoePacked(FMT[self.fmt], self.E, self.N, self.K, self.codes.data_ptr(),
                         self.scales.data_ptr() if self.scales.numel() else 0,
                         0 if self.tensor_scale is None else self.tensor_scale.data_ptr())

    def nbytes(self) -> int:
        n = self.codes.numel() + self.scales.numel()
        return n + (0 if self.tensor_scale is None else 4 * self.tensor_scale.numel())


def _bf16_view(t: torch.Tensor) -> torch.Tensor:
    assert t.element_size() == 2 and t.is_cuda and t.is_contiguous()
    return t


def quantize_weights(fmt: str, w: torch.Tensor, out: PackedWeights | None = None) -> PackedWeights:
    """bf16 masters w [E, N, K] (device) -> PackedWeights (moe_quantize_weights); "w4a16"
    gives the NVFP4 packing its layers use."""
    if fmt == "w4a16":
        fmt = "nvfp4"
    w = _bf16_view(w)
    E, N, K = w.shape
    if out is None:
        out = PackedWeights.empty(fmt, E, N, K, device=w.device)
    st = out.struct()
    _check(lib().moe_quantize_weights(_ptr(w), ctypes.byref(st), _stream(w.device)), "moe_quantize_weights")
    return out


def pack_weights(fmt: str, codes: torch.Tensor, scales: torch.Tensor | None = None,
                 tensor_scale: torch.Tensor | None = None, out: PackedWeights | None = None) -> PackedWeights:
    """Pre-quantised row-major weights (device tensors: codes [E, N, K/2] NVFP4 / MXFP4,
    [E, N, K] MXFP8 and FP8 (uint8) or bf16 (2-byte); scales [E, N, K/16 or K/32]; NVFP4
    tensor scales [E], FP8 channel scales [E, N]) -> PackedWeights (moe_pack_weights);
    "w4a16" packs as NVFP4."""
    if fmt == "w4a16":
        fmt = "nvfp4"
    E, N = codes.shape[0], codes.shape[1]
    K = codes.shape[2] * (2 if fmt in ("nvfp4", "mxfp4") else 1)
    if out is None:
        out = PackedWeights.empty(fmt, E, N, K, device=codes.device)
    src = MoeRowMajor(FMT[fmt], E, N, K, codes.data_ptr(), None if scales is None else scales.data_ptr(),
                      None if tensor_scale is None else tensor_scale.data_ptr())
    st = out.struct()
    _check(lib().moe_pack_weights(ctypes.byref(src), ctypes.byref(st), _stream(codes.device)), "moe_pack_weights")
    return out


def route_workspace(T: int, D: int, E: int, device="cuda") -> torch.Tensor:
    """Device scratch for moe_route over T tokens (reusable across calls of that size)."""
    n = int(lib().moe_route_workspace_bytes(T, D, E))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def route(h: torch.Tensor, wr: torch.Tensor, top_k: int = 8, bias: torch.Tensor | None = None,
          want_amax: bool = False, want_logits: bool = False, workspace: torch.Tensor | None = None):
    """Router (moe_route) -> (topk_idx int32 [T,k], topk_w fp32 [T,k], logits fp32 [T,E] | None,
    h_amax | None). Logits are computed in full only when want_logits is set."""
    h, wr = _bf16_view(h), _bf16_view(wr)
    T, D = h.shape
    E = wr.shape[0]
    dev = h.device
    idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    amax = torch.empty(4, dtype=torch.float32, device=dev) if want_amax else None
    if workspace is None:
        workspace = route_workspace(T, D, E, dev)
    _check(lib().moe_route(T, D, E, top_k, _ptr(h), _ptr(wr), _ptr(bias), _ptr(logits), _ptr(idx), _ptr(w),
                           _ptr(amax), _ptr(workspace), workspace.numel(), _stream(dev)), "moe_route")
    return idx, w, logits, amax


class Layer:
    """Arguments of one moe_forward call, with its workspace and optional taps kept alive."""

    def __init__(self, fmt: str, T: int, D: int, F: int, E: int, gate_up: PackedWeights, down: PackedWeights,
                 top_k: int = 8, e_begin: int = 0, e_end: int | None = None, device="cuda", flags: int = 0):
        self.fmt, self.T, self.D, self.F, self.E, self.top_k = fmt, T, D, F, E, top_k
        self.e_begin, self.e_end = e_begin, E if e_end is None else e_end
        self.gate_up, self.down, self.device = gate_up, down, torch.device(device)
        self.args = MoeForwardArgs()
        a = self.args
        a.fmt, a.T, a.D, a.F, a.E, a.top_k = FMT[fmt], T, D, F, E, top_k
        a.e_begin, a.e_end, a.flags = self.e_begin, self.e_end, flags
        a.gate_up, a.down = gate_up.struct(), down.struct()
        self.workspace_bytes = int(lib().moe_forward_workspace_bytes(ctypes.byref(a)))
        if T > 0 and self.workspace_bytes == 0:
            _check(lib().moe_forward_validate(ctypes.byref(a)), "moe_forward_validate")
        self.workspace = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=self.device)
        a.workspace, a.workspace_bytes = self.workspace.data_ptr(), self.workspace_bytes
        self._taps = None
        self._tap_tensors: dict = {}

    def enable_taps(self):
        """Allocate every debug output of moe_forward (sized for S <= T*top_k). W4A16 has no
        hidden-state codes and its intermediate codes are bf16 bit patterns (int16); FP8 has
        row scales (a_tscale [T], inter_tscale [T*top_k]) instead of block scales."""
        T, D, F, k, n = self.T, self.D, self.F, self.top_k, self.e_end - self.e_begin
        nv, dev = self.fmt == "nvfp4", self.device
        TK = T * k
        spec = {
            "counts": ((n,), torch.int32), "offsets": ((n + 1,), torch.int32),
            "sorted_slot": ((TK,), torch.int32),
            "inter": ((TK, F), torch.float32),
            "y": ((TK, D), torch.float32),
        }
        if self.fmt in ("w4a16", "bf16"):
            spec["inter_codes"] = ((TK, F), torch.int16)
        elif self.fmt == "fp8":
            spec.update({"a_codes": ((T, D), torch.uint8), "inter_codes": ((TK, F), torch.uint8),
                         "a_tscale": ((T,), torch.float32), "inter_tscale": ((TK,), torch.float32)})
        else:
            spec.update({
                "a_codes": ((T, D if self.fmt == "mxfp8" else D // 2), torch.uint8),
                "a_scales": ((T, D // 16 if nv else D // 32), torch.uint8),
                "inter_codes": ((TK, F if self.fmt == "mxfp8" else F // 2), torch.uint8),
                "inter_scales": ((TK, F // 16 if nv else F // 32), torch.uint8),
            })
        if nv:
            spec["a_tscale"] = ((4,), torch.float32)
            spec["inter_tscale"] = ((4,), torch.float32)
        self._tap_tensors = {k_: torch.zeros(s, dtype=d, device=dev) for k_, (s, d) in spec.items()}
        taps = MoeTaps()
        for k_, t in self._tap_tensors.items():
            setattr(taps, k_, t.data_ptr())
        self._taps = taps
        self.args.taps = ctypes.pointer(taps)
        return self._tap_tensors

    def forward(self, h: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                out: torch.Tensor | None = None, h_amax: torch.Tensor | None = None,
                events=None) -> torch.Tensor:
        """moe_forward on the current stream -> out fp32 [T, D]. events: None or a ctypes
        array of N_EVENTS hipEvent_t handles recorded at the stage boundaries."""
        a = self.args
        a.events = None if events is None else ctypes.cast(events, ctypes.c_void_p)
        if out is None:
            out = torch.empty((self.T, self.D), dtype=torch.float32, device=self.device)
        a.h, a.topk_idx, a.topk_w, a.out = h.data_ptr(), topk_idx.data_ptr(), topk_w.data_ptr(), out.data_ptr()
        a.h_amax = None if h_amax is None else h_amax.data_ptr()
        _check(lib().moe_forward(ctypes.byref(a), _stream(self.device)), "moe_forward")
        return out

    def forward_static(self, h: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                       out: torch.Tensor | None = None, h_amax: torch.Tensor | None = None) -> torch.Tensor:
        """moe_forward_static on the current stream (the library's static scratch instead of
        this layer's workspace) -> out fp32 [T, D]."""
        a = MoeForwardArgs.from_buffer_copy(self.args)
        a.workspace, a.workspace_bytes, a.events, a.taps = None, 0, None, None
        if out is None:
            out = torch.empty((self.T, self.D), dtype=torch.float32, device=self.device)
        a.h, a.topk_idx, a.topk_w, a.out = h.data_ptr(), topk_idx.data_ptr(), topk_w.data_ptr(), out.data_ptr()
        a.h_amax = None if h_amax is None else h_amax.data_ptr()
        _check(lib().moe_forward_static(ctypes.byref(a), _stream(self.device)), "moe_forward_static")
        return out

    @property
    def taps(self) -> dict:
        return self._tap_tensors

    def plan(self) -> dict:
        """moe_forward_plan: the kernel family of each GEMM, M-tile rows, workspace bytes."""
        info = MoePlanInfo()
        _check(lib().moe_forward_plan(ctypes.byref(self.args), ctypes.byref(info)), "moe_forward_plan")
        return {"gate_up_kernel": info.gate_up_kernel.decode(), "down_kernel": info.down_kernel.decode(),
                "m_tile_rows": int(info.m_tile_rows), "workspace_bytes": int(info.workspace_bytes)}
