"""CPU oracle of the routed-expert MoE layer (NVFP4 / MXFP8 / MXFP4 experts, NVFP4
weights with bf16 activations, "w4a16", bf16 experts, and FP8 experts with a scale per
weight channel and a dynamic scale per activation row, "fp8").

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and
by bench.py's cpu_baseline leg, never by the library. It wraps oracle.c (plain
C, fp64 expert arithmetic, OpenMP) through ctypes; it shares no code with the
HIP path.

Parity unpinned: the gate-weight exp, the SwiGLU exp and the order of the
fp64 sums are fixed by this specification only (libm accuracy), not by an
external reference.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB selects another build of oracle.c (the sanitizer build of build_sanitized())
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

FMT_NONE, FMT_NVFP4, FMT_MXFP8, FMT_MXFP4, FMT_W4A16, FMT_BF16, FMT_FP8 = 0, 1, 2, 3, 4, 5, 6
# "none": the textbook layer in fp64 on the bf16 masters; "bf16": bf16 experts with the
# GPU's roundings (fp32 sums, bf16 intermediate)
_FMT = {"none": 0, "nvfp4": 1, "mxfp8": 2, "mxfp4": 3, "w4a16": 4, "bf16": 5, "fp8": 6}


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def build_sanitized(path: str) -> str:
    """oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (every UB report fatal),
    for loading through ORACLE_LIB in a process started with the ASan runtime preloaded."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-Wall",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           os.path.join(_HERE, "oracle.c"), "-o", path, "-lm"]
    subprocess.run(cmd, check=True)
    return path


class _Args(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
        ("F", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
        ("e_begin", ctypes.c_int32), ("e_end", ctypes.c_int32),
        ("h", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("gu_master", ctypes.c_void_p), ("dn_master", ctypes.c_void_p),
        ("gu_codes", ctypes.c_void_p), ("gu_scales", ctypes.c_void_p), ("gu_tscale", ctypes.c_void_p),
        ("dn_codes", ctypes.c_void_p), ("dn_scales", ctypes.c_void_p), ("dn_tscale", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("a_codes", ctypes.c_void_p), ("a_scales", ctypes.c_void_p), ("a_tscale", ctypes.c_void_p),
        ("inter", ctypes.c_void_p), ("inter_codes", ctypes.c_void_p),
        ("inter_scales", ctypes.c_void_p), ("inter_tscale", ctypes.c_void_p),
        ("y", ctypes.c_void_p), ("inter_abs", ctypes.c_void_p),
        ("tok_list", ctypes.c_void_p), ("n_tok", ctypes.c_int32),
    ]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, p, dbl, flt = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_float
    lib.orc_e2m1_value.argtypes = [ctypes.c_int]
    lib.orc_e2m1_value.restype = dbl
    lib.orc_e4m3_value.argtypes = [ctypes.c_int]
    lib.orc_e4m3_value.restype = dbl
    lib.orc_e8m0_value.argtypes = [ctypes.c_int]
    lib.orc_e8m0_value.restype = dbl
    lib.orc_e2m1_encode.argtypes = [dbl]
    lib.orc_e2m1_encode.restype = ctypes.c_int
    lib.orc_e4m3_encode.argtypes = [dbl]
    lib.orc_e4m3_encode.restype = ctypes.c_int
    lib.orc_e8m0_code_for_amax.argtypes = [flt]
    lib.orc_e8m0_code_for_amax.restype = ctypes.c_int
    lib.orc_nvfp4_tensor_scale.argtypes = [flt]
    lib.orc_nvfp4_tensor_scale.restype = flt
    lib.orc_quant_nvfp4_mode.argtypes = [p, i64, i64, ctypes.c_int, p, p, p, p]
    lib.orc_quant_nvfp4_mode.restype = ctypes.c_int
    lib.orc_quant_mxfp8.argtypes = [p, i64, i64, p, p]
    lib.orc_quant_mxfp8.restype = ctypes.c_int
    lib.orc_quant_mxfp4.argtypes = [p, i64, i64, p, p]
    lib.orc_quant_mxfp4.restype = ctypes.c_int
    lib.orc_dequant_mxfp4.argtypes = [p, p, i64, i64, p]
    lib.orc_dequant_mxfp4.restype = ctypes.c_int
    lib.orc_mxfp4_scale_code.argtypes = [flt]
    lib.orc_mxfp4_scale_code.restype = ctypes.c_int
    lib.orc_dequant_nvfp4.argtypes = [p, p, flt, i64, i64, ctypes.c_int, p]
    lib.orc_dequant_nvfp4.restype = ctypes.c_int
    lib.orc_dequant_mxfp8.argtypes = [p, p, i64, i64, p]
    lib.orc_dequant_mxfp8.restype = ctypes.c_int
    lib.orc_round_bf16.argtypes = [p, i64, p]
    lib.orc_round_bf16.restype = ctypes.c_int
    lib.orc_quantize_weights.argtypes = [ctypes.c_int, i32, i32, i32, p, p, p, p]
    lib.orc_quantize_weights.restype = ctypes.c_int
    lib.orc_route.argtypes = [i32, i32, i32, i32, p, p, p, p, p, p]
    lib.orc_route.restype = ctypes.c_int
    lib.orc_permute.argtypes = [i32, i32, p, i32, i32, p, p, p]
    lib.orc_permute.restype = i64
    lib.orc_moe_forward.argtypes = [ctypes.POINTER(_Args)]
    lib.orc_moe_forward.restype = ctypes.c_int
    lib.orc_down_combine.argtypes = [i32] * 8 + [p, p, p, p, flt, p, p, p, p, p]
    lib.orc_fp8_row_scale.argtypes = [flt]
    lib.orc_fp8_row_scale.restype = flt
    lib.orc_quant_fp8_rows.argtypes = [p, i64, i64, p, p]
    lib.orc_quant_fp8_rows.restype = ctypes.c_int
    lib.orc_dequant_fp8_rows.argtypes = [p, p, i64, i64, ctypes.c_int, p]
    lib.orc_dequant_fp8_rows.restype = ctypes.c_int
    lib.orc_down_combine.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


# ---------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e8m0_value(code: int) -> float:
    return _load().orc_e8m0_value(int(code))


def e2m1_encode(v: float) -> int:
    return _load().orc_e2m1_encode(float(v))


def e4m3_encode(v: float) -> int:
    return _load().orc_e4m3_encode(float(v))


def e8m0_code_for_amax(amax: float) -> int:
    return _load().orc_e8m0_code_for_amax(float(amax))


def mxfp4_scale_code(amax: float) -> int:
    return _load().orc_mxfp4_scale_code(float(amax))


def nvfp4_tensor_scale(amax: float) -> float:
    return float(_load().orc_nvfp4_tensor_scale(float(amax)))


# ---------------------------------------------------------------- quantisers
NVFP4_RULE = {"4or6": 0, "6": 1, "4": 2}


def quant_nvfp4(x: np.ndarray, with_choice: bool = False, rule: str = "4or6"):
    """NVFP4 of a [rows, K] fp32 tensor as ONE tensor -> (codes [rows,K/2], scales [rows,K/16],
    tensor_scale float32[, chose4 [rows,K/16]]). rule: "4or6" (the layer's quantiser),
    "6" (plain max->6 NVFP4) or "4" (always max->4)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    ch = np.empty((rows, K // 16), np.uint8) if with_choice else None
    _check(_load().orc_quant_nvfp4_mode(_ptr(x), rows, K, NVFP4_RULE[rule], _ptr(codes), _ptr(scales),
                                         _ptr(ts), _ptr(ch)), "quant_nvfp4")
    return (codes, scales, ts[0], ch) if with_choice else (codes, scales, ts[0])


def quant_mxfp8(x: np.ndarray):
    """MXFP8 of a [rows, K] fp32 tensor -> (codes [rows,K], scales [rows,K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    _check(_load().orc_quant_mxfp8(_ptr(x), rows, K, _ptr(codes), _ptr(scales)), "quant_mxfp8")
    return codes, scales


def fp8_row_scale(amax: float) -> float:
    """The FP8 row scale for a row whose largest magnitude is amax (fp32)."""
    return float(_load().orc_fp8_row_scale(amax))


def quant_fp8_rows(x: np.ndarray):
    """E4M3 with one fp32 scale per row of a [rows, K] fp32 tensor -> (codes [rows,K],
    scales float32 [rows])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty(rows, np.float32)
    _check(_load().orc_quant_fp8_rows(_ptr(x), rows, K, _ptr(codes), _ptr(scales)), "quant_fp8_rows")
    return codes, scales


def dequant_fp8_rows(codes, scales=None) -> np.ndarray:
    """codes [rows, K] -> fp64 values, times the row scales when given."""
    codes = np.ascontiguousarray(codes, np.uint8)
    rows, K = codes.shape
    sc = None if scales is None else np.ascontiguousarray(scales, np.float32)
    out = np.empty((rows, K), np.float64)
    _check(_load().orc_dequant_fp8_rows(_ptr(codes), _ptr(sc), rows, K, 0 if sc is None else 1, _ptr(out)),
           "dequant_fp8_rows")
    return out


def dequant_nvfp4(codes, scales, tensor_scale, with_tensor=True) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, K), np.float64)
    _check(_load().orc_dequant_nvfp4(_ptr(codes), _ptr(scales), float(tensor_scale), rows, K,
                                     1 if with_tensor else 0, _ptr(out)), "dequant_nvfp4")
    return out


def quant_mxfp4(x: np.ndarray):
    """MXFP4 of a [rows, K] fp32 tensor -> (codes [rows,K/2] (element 2i in the low
    nibble), scales [rows,K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    _check(_load().orc_quant_mxfp4(_ptr(x), rows, K, _ptr(codes), _ptr(scales)), "quant_mxfp4")
    return codes, scales


def dequant_mxfp4(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, K), np.float64)
    _check(_load().orc_dequant_mxfp4(_ptr(codes), _ptr(scales), rows, K, _ptr(out)), "dequant_mxfp4")
    return out


def dequant_mxfp8(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, K = codes.shape
    out = np.empty((rows, K), np.float64)
    _check(_load().orc_dequant_mxfp8(_ptr(codes), _ptr(scales), rows, K, _ptr(out)), "dequant_mxfp8")
    return out


def fold_to_mx(values: np.ndarray, fmt: str = "mxfp8") -> np.ndarray:
    """The values a scaled MFMA that takes one E8M0 scale per 32 values would see if exact
    values [rows, K] (e.g. NVFP4 codes times their per-16 E4M3 block scales, each exact in
    fp32) were folded into its operands: each 32-block re-encoded by the OCP MX rule (E8M0
    scale 2^(floor(log2 amax) - 8) for E4M3 elements, - 2 for E2M1, elements rounded to
    nearest even, saturating), fp64. Test-side emulation of the alternative to the exact
    16-bit expansion; the MX quantisers and dequantisers below do the work."""
    x = np.ascontiguousarray(values, np.float32)
    assert np.array_equal(x.astype(np.float64), np.asarray(values, np.float64)), "values must be exact in fp32"
    if fmt == "mxfp8":
        return dequant_mxfp8(*quant_mxfp8(x))
    if fmt == "mxfp4":
        return dequant_mxfp4(*quant_mxfp4(x))
    raise ValueError(fmt)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), nearest with ties to even."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _check(_load().orc_round_bf16(_ptr(x), x.size, _ptr(out)), "round_bf16")
    return out


def quantize_weights(fmt: str, w_bf16: np.ndarray):
    """Quantise bf16 masters [E, N, K] per expert -> dict(codes, scales, tensor_scale|None).
    W4A16 weights are NVFP4 weights; FP8 weights have no block scales (scales None) and one
    fp32 scale per output channel (tensor_scale [E, N])."""
    f = _FMT[fmt]
    if f == FMT_W4A16:
        f = FMT_NVFP4
    w = np.ascontiguousarray(w_bf16, np.uint16)
    E, N, K = w.shape
    if f == FMT_NVFP4:
        codes = np.empty((E, N, K // 2), np.uint8)
        scales = np.empty((E, N, K // 16), np.uint8)
        ts = np.empty(E, np.float32)
    elif f == FMT_MXFP4:
        codes = np.empty((E, N, K // 2), np.uint8)
        scales = np.empty((E, N, K // 32), np.uint8)
        ts = None
    elif f == FMT_FP8:
        codes = np.empty((E, N, K), np.uint8)
        scales = None
        ts = np.empty((E, N), np.float32)
    else:
        codes = np.empty((E, N, K), np.uint8)
        scales = np.empty((E, N, K // 32), np.uint8)
        ts = None
    _check(_load().orc_quantize_weights(f, E, N, K, _ptr(w), _ptr(codes), _ptr(scales), _ptr(ts)),
           "quantize_weights")
    return {"codes": codes, "scales": scales, "tensor_scale": ts}


# ---------------------------------------------------------------- router / permute
def route(h_bf16: np.ndarray, wr_bf16: np.ndarray, k: int = 8, bias: np.ndarray | None = None,
          want_logits: bool = False):
    """Softmax-then-top-k router -> (idx int32 [T,k], w float32 [T,k][, logits float32 [T,E]])."""
    h = np.ascontiguousarray(h_bf16, np.uint16)
    wr = np.ascontiguousarray(wr_bf16, np.uint16)
    T, D = h.shape
    E = wr.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lg = np.empty((T, E), np.float32) if want_logits else None
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    _check(_load().orc_route(T, D, E, k, _ptr(h), _ptr(wr), _ptr(b), _ptr(idx), _ptr(w), _ptr(lg)),
           "route")
    return (idx, w, lg) if want_logits else (idx, w)


def permute(idx: np.ndarray, e_begin: int, e_end: int):
    """-> (counts [n], offsets [n+1], sorted_slot [S]) for local experts [e_begin, e_end)."""
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    n = e_end - e_begin
    counts = np.empty(n, np.int32)
    offs = np.empty(n + 1, np.int32)
    sorted_slot = np.empty(T * k, np.int32)
    S = _load().orc_permute(T, k, _ptr(idx), e_begin, e_end, _ptr(counts), _ptr(offs), _ptr(sorted_slot))
    if S < 0:
        raise RuntimeError(f"oracle permute failed ({S})")
    return counts, offs, sorted_slot[:S].copy()


# ---------------------------------------------------------------- layer
def moe_forward(fmt: str, h_bf16, idx, w, *, D: int, F: int, E: int, e_begin: int = 0,
                e_end: int | None = None, gate_up=None, down=None, gate_up_master=None,
                down_master=None, taps: bool = False, tok_list=None):
    """Oracle MoE forward -> out float32 [T, D] (and a dict of taps when taps=True).

    gate_up/down: dicts from quantize_weights (fmt nvfp4/mxfp8/mxfp4/w4a16/fp8); *_master: bf16
    arrays (fmt none and bf16). FP8 taps: a_tscale [T] and inter_tscale [S] are the row scales.
    tok_list: compute only these tokens' outputs (others are zero)."""
    f = _FMT[fmt]
    lib = _load()
    h = np.ascontiguousarray(h_bf16, np.uint16)
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T, k = idx.shape
    e_end = E if e_end is None else e_end
    out = np.empty((T, D), np.float32)
    keep = []  # arrays that must outlive the call
    a = _Args()
    a.fmt, a.T, a.D, a.F, a.E, a.k, a.e_begin, a.e_end = f, T, D, F, E, k, e_begin, e_end
    a.h, a.idx, a.w, a.out = _ptr(h), _ptr(idx), _ptr(w), _ptr(out)
    if f in (FMT_NONE, FMT_BF16):
        gm = np.ascontiguousarray(gate_up_master, np.uint16)
        dm = np.ascontiguousarray(down_master, np.uint16)
        keep += [gm, dm]
        a.gu_master, a.dn_master = _ptr(gm), _ptr(dm)
    else:
        for name, d in (("gu", gate_up), ("dn", down)):
            c = np.ascontiguousarray(d["codes"], np.uint8)
            s = None if d.get("scales") is None else np.ascontiguousarray(d["scales"], np.uint8)
            ts = None if d.get("tensor_scale") is None else np.ascontiguousarray(d["tensor_scale"], np.float32)
            keep += [c, s, ts]
            setattr(a, f"{name}_codes", _ptr(c))
            setattr(a, f"{name}_scales", _ptr(s))
            setattr(a, f"{name}_tscale", _ptr(ts))
    tp = {}
    if taps:
        _, offs, _ = permute(idx, e_begin, e_end)
        S = int(offs[-1])
        if f in (FMT_W4A16, FMT_BF16):
            # no activation codes; the intermediate is bf16 bit patterns [S][F]
            tp["inter"] = np.zeros((S, F), np.float32)
            tp["inter_codes"] = np.zeros((S, F), np.uint16)
            a.inter, a.inter_codes = _ptr(tp["inter"]), _ptr(tp["inter_codes"])
        elif f == FMT_FP8:
            tp["a_codes"] = np.zeros((T, D), np.uint8)
            tp["a_tscale"] = np.zeros(T, np.float32)
            tp["inter"] = np.zeros((S, F), np.float32)
            tp["inter_codes"] = np.zeros((S, F), np.uint8)
            tp["inter_tscale"] = np.zeros(S, np.float32)
            for n in ("a_codes", "a_tscale", "inter", "inter_codes", "inter_tscale"):
                setattr(a, n, _ptr(tp[n]))
        elif f != FMT_NONE:
            tp["a_codes"] = np.zeros((T, D if f == FMT_MXFP8 else D // 2), np.uint8)
            tp["a_scales"] = np.zeros((T, D // 16 if f == FMT_NVFP4 else D // 32), np.uint8)
            tp["a_tscale"] = np.zeros(1, np.float32)
            tp["inter"] = np.zeros((S, F), np.float32)
            tp["inter_codes"] = np.zeros((S, F if f == FMT_MXFP8 else F // 2), np.uint8)
            tp["inter_scales"] = np.zeros((S, F // 16 if f == FMT_NVFP4 else F // 32), np.uint8)
            tp["inter_tscale"] = np.zeros(1, np.float32)
            for n in ("a_codes", "a_scales", "a_tscale", "inter", "inter_codes", "inter_scales",
                      "inter_tscale"):
                setattr(a, n, _ptr(tp[n]))
        tp["y"] = np.zeros((S, D), np.float32)
        tp["inter_abs"] = np.zeros((S, 2 * F), np.float64)
        a.y, a.inter_abs = _ptr(tp["y"]), _ptr(tp["inter_abs"])
    if tok_list is not None:
        tl = np.ascontiguousarray(tok_list, np.int32)
        keep.append(tl)
        a.tok_list, a.n_tok = _ptr(tl), len(tl)
    _check(lib.orc_moe_forward(ctypes.byref(a)), "moe_forward")
    return (out, tp) if taps else out


def down_combine(fmt: str, idx, w, inter_codes, inter_scales, inter_tscale, down, *, D: int, F: int, E: int,
                 e_begin: int = 0, e_end: int | None = None):
    """Down projection and combine alone (the forward's last two steps) from given
    intermediate codes of the S local slots in sorted order -> out float32 [T, D].
    W4A16: inter_codes are bf16 bit patterns [S][F] and inter_scales is None. FP8:
    inter_codes are E4M3 [S][F] and inter_tscale is the row scales [S]."""
    f = _FMT[fmt]
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T, k = idx.shape
    e_end = E if e_end is None else e_end
    ic = np.ascontiguousarray(inter_codes, np.uint16 if f in (FMT_W4A16, FMT_BF16) else np.uint8)
    is_ = None if inter_scales is None else np.ascontiguousarray(inter_scales, np.uint8)
    if f == FMT_BF16:  # down is the bf16 master [E][D][F]
        c, sc = np.ascontiguousarray(down, np.uint16), None
    else:
        c = np.ascontiguousarray(down["codes"], np.uint8)
        sc = None if down.get("scales") is None else np.ascontiguousarray(down["scales"], np.uint8)
    ts = (None if f == FMT_BF16 or down.get("tensor_scale") is None
          else np.ascontiguousarray(down["tensor_scale"], np.float32))
    rs = None
    if f == FMT_FP8:
        rs = np.ascontiguousarray(inter_tscale, np.float32)
        inter_tscale = None
    out = np.empty((T, D), np.float32)
    _check(_load().orc_down_combine(f, T, D, F, E, k, e_begin, e_end, _ptr(idx), _ptr(w), _ptr(ic), _ptr(is_),
                                    float(inter_tscale if inter_tscale is not None else 1.0), _ptr(c), _ptr(sc),
                                    _ptr(ts), _ptr(rs), _ptr(out)), "down_combine")
    return out
