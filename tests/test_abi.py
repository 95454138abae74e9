"""The C ABI on the host (no GPU needed): the library loads, exports every function
include/moe.h declares, and its host-side validation returns the documented status
codes before anything is enqueued."""
import ctypes
import os
import re

import pytest

import block_scaled_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, EINVAL, EUNSUP, EALIGN, EWS = 0, -1, -2, -3, -4
A16 = 0x10000  # a fake, 16-byte aligned "device" address: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_functions_are_exported_and_bound():
    lib = moe.lib()
    names = declared_functions()
    assert len(names) == 11, names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported by libmoe.so"
        assert n in moe.SIGNATURES, f"{n} has no binding"
    assert lib.moe_abi_version() == 8
    assert lib.moe_status_string(EWS) == b"workspace missing or too small"


def _args(**over):
    a = moe.MoeForwardArgs()
    a.fmt, a.T, a.D, a.F, a.E, a.top_k, a.e_begin, a.e_end = 1, 64, 4096, 2560, 384, 8, 0, 384
    a.h = a.topk_idx = a.topk_w = a.out = A16
    a.gate_up = moe.MoePacked(1, 384, 5120, 4096, A16, A16, A16)
    a.down = moe.MoePacked(1, 384, 4096, 2560, A16, A16, A16)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _validate(a):
    return moe.lib().moe_forward_validate(ctypes.byref(a))


def test_forward_validation_accepts_the_workloads():
    assert _validate(_args()) == OK
    mx = _args(fmt=2)
    mx.gate_up = moe.MoePacked(2, 384, 5120, 4096, A16, A16, 0)
    mx.down = moe.MoePacked(2, 384, 4096, 2560, A16, A16, 0)
    assert _validate(mx) == OK
    m4 = _args(fmt=3)
    m4.gate_up = moe.MoePacked(3, 384, 5120, 4096, A16, A16, 0)
    m4.down = moe.MoePacked(3, 384, 4096, 2560, A16, A16, 0)
    assert _validate(m4) == OK
    assert _validate(_args(fmt=4)) == OK  # W4A16 on NVFP4-packed weights
    b16 = _args(fmt=5)
    b16.gate_up = moe.MoePacked(5, 384, 5120, 4096, A16, 0, 0)  # bf16 weights: no scales
    b16.down = moe.MoePacked(5, 384, 4096, 2560, A16, 0, 0)
    assert _validate(b16) == OK
    assert _validate(_fp8()) == OK
    assert _validate(_args(T=0, h=0, topk_idx=0, topk_w=0, out=0)) == OK  # empty batch


def _fp8(**over):
    """FP8 layer: E4M3 codes, no block scales, channel scales in tensor_scale."""
    a = _args(fmt=6, **over)
    a.gate_up = moe.MoePacked(6, a.E, 2 * a.F, a.D, A16, 0, A16)
    a.down = moe.MoePacked(6, a.E, a.D, a.F, A16, 0, A16)
    return a


def test_fp8_layer_host_checks():
    lib = moe.lib()
    a = _fp8()
    a.gate_up = moe.MoePacked(6, 384, 5120, 4096, A16, 0, 0)    # channel scales missing
    assert _validate(a) == EINVAL
    assert _validate(_fp8(flags=moe.FLAG_EXACT_SUMS)) == EUNSUP  # no exact-sum route
    assert _validate(_fp8(D=384)) == EUNSUP                       # 256-row weight tiles of the scaled MFMA
    info = moe.MoePlanInfo()
    assert lib.moe_forward_plan(ctypes.byref(_fp8()), ctypes.byref(info)) == OK
    assert info.gate_up_kernel == b"mx_gemm_kernel" and info.down_kernel == b"mx_gemm_kernel"
    # fp32 row scales of the hidden states and of the slots, and the fp32 intermediate
    ws = lib.moe_forward_workspace_bytes
    assert ws(ctypes.byref(_fp8())) > 64 * 8 * 2560 * 4 + 64 * 8 * 4096 * 4
    # quantise / pack: FP8 takes no block scales but needs the channel scales
    p = ctypes.c_void_p
    out = moe.MoePacked(6, 2, 64, 128, A16, 0, 0)
    assert lib.moe_quantize_weights(p(A16), ctypes.byref(out), None) == EINVAL
    src = moe.MoeRowMajor(6, 2, 64, 128, A16, 0, 0)
    out = moe.MoePacked(6, 2, 64, 128, A16, 0, A16)
    assert lib.moe_pack_weights(ctypes.byref(src), ctypes.byref(out), None) == EINVAL
    src = moe.MoeRowMajor(6, 2, 64, 128, A16, 0, A16 + 2)
    assert lib.moe_pack_weights(ctypes.byref(src), ctypes.byref(out), None) == EALIGN


def test_w4a16_takes_nvfp4_packed_weights():
    a = _args(fmt=4)
    a.gate_up = moe.MoePacked(4, 384, 5120, 4096, A16, A16, A16)   # the packing is NVFP4's
    assert _validate(a) == EINVAL
    a = _args(fmt=4)
    a.down = moe.MoePacked(1, 384, 4096, 2560, A16, A16, 0)        # NVFP4 needs its tensor scales
    assert _validate(a) == EINVAL


def test_mxfp4_needs_256_wide_d_model():
    m4 = _args(fmt=3, D=384)
    m4.gate_up = moe.MoePacked(3, 384, 5120, 384, A16, A16, 0)
    m4.down = moe.MoePacked(3, 384, 384, 2560, A16, A16, 0)
    assert _validate(m4) == EUNSUP


def test_scaled_mfma_row_scale_limit():
    """The MX kernel stages each activation row's E8M0 scales for the whole K in LDS, so
    MXFP4 takes K <= 8192 (D and F); MXFP8 beyond it runs the exact route; FP8 (one scale
    per row) has no such limit."""
    def m4(D, F):
        a = _args(fmt=3, D=D, F=F)
        a.gate_up = moe.MoePacked(3, 384, 2 * F, D, A16, A16, 0)
        a.down = moe.MoePacked(3, 384, D, F, A16, A16, 0)
        return a
    assert _validate(m4(8192, 2560)) == OK
    assert _validate(m4(8448, 2560)) == EUNSUP
    assert _validate(m4(4096, 8320)) == EUNSUP
    a = _mx8(T=16384, D=8448)
    a.gate_up = moe.MoePacked(2, 384, 5120, 8448, A16, A16, 0)
    a.down = moe.MoePacked(2, 384, 8448, 2560, A16, A16, 0)
    rc, info = _plan(a)
    assert rc == OK and info.gate_up_kernel == b"tile_gemm_kernel"
    f = _fp8(D=8448)
    assert _validate(f) == OK and _plan(f)[1].gate_up_kernel == b"mx_gemm_kernel"


@pytest.mark.parametrize("over,status", [
    (dict(fmt=7), EINVAL), (dict(fmt=0), EINVAL), (dict(T=-1), EINVAL), (dict(top_k=0), EINVAL), (dict(top_k=9), EINVAL),
    (dict(e_begin=10, e_end=10), EINVAL), (dict(e_end=385), EINVAL), (dict(e_begin=-1), EINVAL),
    (dict(E=5000), EINVAL), (dict(h=0), EINVAL), (dict(out=0), EINVAL),
    (dict(D=4000), EUNSUP), (dict(F=2500), EUNSUP),
    (dict(h=A16 + 2), EALIGN), (dict(out=A16 + 4), EALIGN), (dict(topk_w=A16 + 8), EALIGN),
])
def test_forward_validation_rejects(over, status):
    assert _validate(_args(**over)) == status


def test_packed_weights_must_match_the_layer():
    a = _args()
    a.gate_up = moe.MoePacked(1, 384, 5120, 2048, A16, A16, A16)  # K != D
    assert _validate(a) == EINVAL
    a = _args()
    a.down = moe.MoePacked(2, 384, 4096, 2560, A16, A16, A16)  # format mismatch
    assert _validate(a) == EINVAL
    a = _args()
    a.gate_up = moe.MoePacked(1, 384, 5120, 4096, A16, A16, 0)  # NVFP4 needs tensor scales
    assert _validate(a) == EINVAL
    a = _args()
    a.down = moe.MoePacked(1, 384, 4096, 2560, A16 + 1, A16, A16)
    assert _validate(a) == EALIGN


def test_forward_rejects_missing_workspace_before_any_launch():
    a = _args()
    assert moe.lib().moe_forward(ctypes.byref(a), None) == EWS
    a.workspace, a.workspace_bytes = A16, 1024
    assert moe.lib().moe_forward(ctypes.byref(a), None) == EWS
    assert moe.lib().moe_forward(ctypes.byref(_args(top_k=9)), None) == EINVAL


def test_workspace_plan_sizes():
    ws = moe.lib().moe_forward_workspace_bytes
    small = ws(ctypes.byref(_args()))
    big = ws(ctypes.byref(_args(T=8192, e_end=96)))
    assert 0 < small < big
    # dominated by the fp32 per-slot down projection y [T*k][D]
    assert big >= 8192 * 8 * 4096 * 4
    assert ws(ctypes.byref(_args(top_k=0))) == 0


def test_route_and_quantize_validate_on_the_host():
    lib = moe.lib()
    p = ctypes.c_void_p
    ws = lib.moe_route_workspace_bytes(4, 64, 16)
    assert ws > 0 and lib.moe_route_workspace_bytes(4, 96, 16) == 0 and lib.moe_route_workspace_bytes(4, 64, 2000) == 0
    r = lambda T, D, E, k, h, ws_ptr, ws_n: lib.moe_route(T, D, E, k, p(h), p(A16), None, None, p(A16), p(A16), None,
                                                          ws_ptr, ws_n, None)
    assert r(4, 64, 16, 9, A16, p(A16), ws) == EINVAL          # top_k > 8
    assert r(4, 96, 16, 8, A16, p(A16), ws) == EUNSUP          # D not a multiple of 64
    assert r(4, 64, 16, 8, A16 + 2, p(A16), ws) == EALIGN      # misaligned h
    assert r(4, 64, 16, 8, A16, p(A16), ws - 1) == EWS         # workspace too small
    assert r(4, 64, 16, 8, A16, None, ws) == EWS               # workspace missing
    assert r(0, 64, 16, 8, 0, None, 0) == OK                   # empty batch: no-op
    # the screened path (from 512 tokens) needs more room than the exact one
    assert lib.moe_route_workspace_bytes(512, 4096, 384) > lib.moe_route_workspace_bytes(511, 4096, 384)
    bad = moe.MoePacked(1, 2, 32, 96, A16, A16, A16)   # K must be a multiple of 64 (tiled layout)
    assert lib.moe_quantize_weights(p(A16), ctypes.byref(bad), None) == EINVAL
    bad = moe.MoePacked(2, 2, 48, 64, A16, A16, 0)     # N must be a multiple of 32 (tiled layout)
    assert lib.moe_quantize_weights(p(A16), ctypes.byref(bad), None) == EINVAL
    bad = moe.MoePacked(1, 2, 32, 64, A16, A16, 0)     # NVFP4 needs the tensor-scale buffer
    assert lib.moe_quantize_weights(p(A16), ctypes.byref(bad), None) == EINVAL
    bad = moe.MoePacked(4, 2, 32, 64, A16, A16, A16)   # unknown format
    assert lib.moe_quantize_weights(p(A16), ctypes.byref(bad), None) == EINVAL
    bad = moe.MoePacked(2, 2, 32, 64, A16 + 8, A16, 0)  # misaligned codes
    assert lib.moe_quantize_weights(p(A16), ctypes.byref(bad), None) == EALIGN


def _plan(a):
    info = moe.MoePlanInfo()
    rc = moe.lib().moe_forward_plan(ctypes.byref(a), ctypes.byref(info))
    return rc, info


def _mx8(**over):
    a = _args(fmt=2, **over)
    a.gate_up = moe.MoePacked(2, 384, 5120, 4096, A16, A16, 0)
    a.down = moe.MoePacked(2, 384, 4096, 2560, A16, A16, 0)
    return a


def test_forward_plan_names_the_kernels():
    """moe_forward_plan reports the dispatch of moe_forward (the same host plan)."""
    rc, info = _plan(_args())                                   # NVFP4 decode: streaming kernels
    assert rc == OK and info.gate_up_kernel == b"stream_gemm_kernel" and info.down_kernel == b"stream_gemm_kernel"
    rc, info = _plan(_args(T=8192, e_end=96))                   # NVFP4 EP4 prefill: MFMA tiles
    assert rc == OK and info.gate_up_kernel == b"tile_gemm_kernel" and info.m_tile_rows == 64
    assert info.workspace_bytes == moe.lib().moe_forward_workspace_bytes(ctypes.byref(_args(T=8192, e_end=96)))
    rc, info = _plan(_mx8(T=16384))                             # MXFP8 prefill: scaled FP8 MFMA
    assert rc == OK and info.gate_up_kernel == b"mx_gemm_kernel" and info.m_tile_rows == 128
    rc, info = _plan(_fp8(T=8192, e_end=96))                    # FP8 prefill: 256 x 256 tiles
    assert rc == OK and info.gate_up_kernel == b"fp8_wide_gemm_kernel" and info.m_tile_rows == 256
    assert info.down_kernel == b"fp8_wide_gemm_kernel"
    rc, info = _plan(_fp8())                                    # FP8 decode: 128-row tiles
    assert rc == OK and info.gate_up_kernel == b"mx_gemm_kernel" and info.m_tile_rows == 128
    rc, info = _plan(_mx8(T=16384, flags=1))                    # exact sums: the bf16 expansion
    assert rc == OK and info.gate_up_kernel == b"tile_gemm_kernel"
    rc, info = _plan(_mx8(T=256, flags=1))
    assert rc == OK and info.gate_up_kernel == b"stream_gemm_kernel"
    # the exact route keeps 16-bit operand copies, the scaled route needs none
    ws = moe.lib().moe_forward_workspace_bytes
    assert ws(ctypes.byref(_mx8(T=16384, flags=1))) > ws(ctypes.byref(_mx8(T=16384)))
    rc, info = _plan(_mx8(T=256, D=384))                        # no 256-wide down blocks: bf16 route
    assert rc == OK and info.gate_up_kernel != b"mx_gemm_kernel"
    assert _plan(_args(flags=2))[0] == EINVAL                   # unknown flag
    assert _validate(_args(flags=2)) == EINVAL
    rc, info = _plan(_args(T=0))
    assert rc == OK and info.gate_up_kernel == b"none"


def test_forward_static_validates_on_the_host():
    """moe_forward_static: the static scratch's limit and the argument checks come first."""
    lib = moe.lib()
    assert lib.moe_forward_static(ctypes.byref(_args(top_k=9)), None) == EINVAL
    assert lib.moe_forward_static(ctypes.byref(_args(h=A16 + 2)), None) == EALIGN
    big = _args(T=8192, e_end=96)   # about 1.4 GB of workspace: beyond the 64 MiB array
    assert moe.lib().moe_forward_workspace_bytes(ctypes.byref(big)) > moe.STATIC_SCRATCH_BYTES
    assert lib.moe_forward_static(ctypes.byref(big), None) == EWS
    assert moe.lib().moe_forward_workspace_bytes(ctypes.byref(_args())) <= moe.STATIC_SCRATCH_BYTES
    mx = _args(fmt=2, T=256)
    mx.gate_up = moe.MoePacked(2, 384, 5120, 4096, A16, A16, 0)
    mx.down = moe.MoePacked(2, 384, 4096, 2560, A16, A16, 0)
    assert moe.lib().moe_forward_workspace_bytes(ctypes.byref(mx)) <= moe.STATIC_SCRATCH_BYTES
    assert lib.moe_forward_static(ctypes.byref(_args(T=0, h=0, topk_idx=0, topk_w=0, out=0)), None) == OK


def test_pack_weights_validates_on_the_host():
    lib = moe.lib()
    p = lambda *a: moe.MoeRowMajor(*a)
    ok_out = moe.MoePacked(1, 2, 64, 128, A16, A16, A16)
    assert lib.moe_pack_weights(None, ctypes.byref(ok_out), None) == EINVAL
    assert lib.moe_pack_weights(ctypes.byref(p(1, 2, 64, 128, A16, A16, 0)), ctypes.byref(ok_out), None) == EINVAL
    assert lib.moe_pack_weights(ctypes.byref(p(2, 2, 64, 128, A16, A16, 0)), ctypes.byref(ok_out), None) == EINVAL
    assert lib.moe_pack_weights(ctypes.byref(p(1, 2, 64, 96, A16, A16, A16)),
                                ctypes.byref(moe.MoePacked(1, 2, 64, 96, A16, A16, A16)), None) == EINVAL
    assert lib.moe_pack_weights(ctypes.byref(p(1, 2, 64, 128, A16 + 8, A16, A16)), ctypes.byref(ok_out),
                                None) == EALIGN
    mx = moe.MoePacked(2, 2, 64, 128, A16, 0, 0)
    assert lib.moe_pack_weights(ctypes.byref(p(2, 2, 64, 128, A16, A16, 0)), ctypes.byref(mx), None) == EINVAL
