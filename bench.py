"""Benchmark of the block-scaled MoE layer on one MI355X.

One step = the whole hot path over one batch: moe_route (router logits, top-8, gate
weights, hidden-state amax) + moe_forward (permutation, hidden-state quantisation,
gate_up GEMM with SwiGLU and intermediate quantisation, down GEMM, weighted
combine), with all inputs and packed weights resident in HBM.

By default the five seeded workloads of the layer's configurations run one after the
other: tiny-nvfp4 (16 tokens, d_model 256), decode-nvfp4 (64 tokens, d_model 4096,
d_ff 2560, 384 experts, top-8), decode-mxfp8 (256 tokens), prefill-nvfp4-ep4 (8192
tokens, one expert-parallel rank's 96 experts) and skewed-mxfp8 (16384 tokens, Zipf-like
router bias). The headline fields of the JSON line are decode-nvfp4's; `configs` holds
every workload's line. --workload i runs one of the thirteen synthetic workloads alone
(the five plus the MXFP4, W4A16, bf16-expert and FP8 variants).

Printed: one JSON line (rank 0). `roofline` covers the dominant kernel (the gate_up
GEMM) timed live with HIP events recorded around its launch on the library's stream;
`cpu_baseline` is the CPU oracle timed on this host's cores over a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "fp8": 5033.2, "fp4": 10066.3}  # dense, MI355X
DTYPES = {"nvfp4": "f16 (exact NVFP4 values), fp32 accumulate",
          "mxfp8": "fp8 (MXFP8 codes and E8M0 scales on the scaled MFMA), fp32 accumulate",
          "mxfp4": "fp4 (MXFP4 codes and E8M0 scales on the scaled MFMA), fp32 accumulate",
          "w4a16": "bf16 (bf16 activations, NVFP4 weights expanded exactly), fp32 accumulate",
          "bf16": "bf16 (bf16 weights and activations), fp32 accumulate",
          "fp8": "fp8 (E4M3 codes on the scaled MFMA with unit scales, fp32 row and channel scales applied "
                 "to the sums), fp32 accumulate"}
METRIC = "MoE layer tokens/s; % peak HBM BW (decode), % scaled-MFMA peak (prefill)"


class HipEvents:
    """Raw hipEvent_t handles (libamdhip64), recorded by the library on its stream."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            self.arr[i] = ev

    def ms(self, i: int, j: int) -> float:
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), self.arr[i], self.arr[j])
        assert rc == 0, f"hipEventElapsedTime failed ({rc})"
        return float(out.value)

    def close(self):
        for i in range(len(self.arr)):
            self.hip.hipEventDestroy(self.arr[i])


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "block_scaled_moe_amd", "csrc")
# sources that decide the code of each gate_up kernel family (a traffic figure measured
# with rocprofv3 is valid only while their hash is unchanged)
KERNEL_SOURCES = {
    "stream_gemm_kernel": ["gemm_stream.hip", "gemm_common.h", "layout.h", "formats.h"],
    "tile_gemm_kernel": ["gemm_tile.hip", "gemm_common.h", "layout.h", "formats.h"],
    "grouped_gemm_kernel": ["gemm.hip", "gemm_common.h", "layout.h", "formats.h"],
    "mx_gemm_kernel": ["gemm_mx.hip", "gemm_common.h", "layout.h", "formats.h"],
    "fp8_wide_gemm_kernel": ["gemm_fp8_wide.hip", "gemm_common.h", "layout.h", "formats.h"],
    "bf16_wide_gemm_kernel": ["gemm_bf16_wide.hip", "gemm_common.h", "layout.h", "formats.h"],
}


def kernel_source_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(workload: str, kernel: str):
    """Calibrated HBM bytes per gate_up launch from profiles/<workload>_gate_up_traffic.md,
    or None if there is no such summary or the kernel's sources changed since."""
    import re
    path = os.path.join(HERE, "profiles", f"{workload}_gate_up_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_k = re.search(r"kernel:\s*(\w+)", text)
    if not (m_b and m_h and m_k) or m_k.group(1) != kernel or m_h.group(1) != kernel_source_hash(kernel):
        return None
    return int(m_b.group(1))


def packed_bytes_per_expert(fmt: str, N: int, K: int) -> int:
    if fmt in ("nvfp4", "w4a16"):
        return N * K // 2 + N * K // 16 + 4
    if fmt == "bf16":
        return 2 * N * K
    if fmt == "mxfp4":
        return N * K // 2 + N * K // 32
    if fmt == "fp8":
        return N * K + 4 * N
    return N * K + N * K // 32


def make_weights(moe, torch, wl, dev):
    """Packed gate_up and down of all experts, masters drawn on the GPU in expert chunks."""
    E, D, F = wl.E, wl.D, wl.F
    gu = moe.PackedWeights.empty(wl.fmt, E, 2 * F, D, device=dev)
    dn = moe.PackedWeights.empty(wl.fmt, E, D, F, device=dev)
    chunk = max(1, min(E, (1 << 30) // (2 * F * D * 2)))
    buf = torch.empty(chunk * 2 * F * D, dtype=torch.int16, device=dev)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        n = e1 - e0
        g = buf[: n * 2 * F * D]
        wl.gate_up_master_device(e0, e1, g)
        moe.quantize_weights(wl.fmt, g.view(n, 2 * F, D), out=gu.experts(e0, e1))
        d = buf[: n * D * F]
        wl.down_master_device(e0, e1, d)
        moe.quantize_weights(wl.fmt, d.view(n, D, F), out=dn.experts(e0, e1))
    torch.cuda.synchronize()
    del buf
    return gu, dn


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, h, wr, bias, target_s: float = 10.0):
    """The oracle (route + forward, fp64 experts) on the first tokens of the workload,
    timed on this host; the sample grows until it takes about target_s seconds.
    Experts are compacted to those the sample touches (weights quantised by the
    oracle itself once per expert, untimed)."""
    import oracle

    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    quantised = {}  # expert -> (gate_up, down) of the oracle's quantiser
    n = 2
    while True:
        hs = np.ascontiguousarray(h[:n])
        t0 = time.perf_counter()
        idx, w = oracle.route(hs, wr, k=wl.k, bias=bias)
        t_route = time.perf_counter() - t0
        local = (idx >= wl.e_begin) & (idx < wl.local_end)
        used = np.unique(idx[local])
        remap = np.full(wl.E, -1, np.int32)
        remap[used] = np.arange(len(used), dtype=np.int32)
        cidx = np.where(local, remap[idx], len(used)).astype(np.int32)  # non-local -> outside [0, m)
        m = len(used)
        if m == 0 and n < wl.T:  # no local slot in the sample yet (an expert-parallel share)
            n = min(wl.T, 2 * n)
            continue
        if wl.fmt == "bf16":  # unquantised: the touched experts' masters plus zero experts
            pad = max(1, wl.k - m)
            z = lambda a: np.concatenate([a, np.zeros((pad,) + a.shape[1:], a.dtype)])
            gm = z(np.stack([wl.gate_up_master(int(e))[0] for e in used]))
            dm = z(np.stack([wl.down_master(int(e))[0] for e in used]))
            t1 = time.perf_counter()
            oracle.moe_forward("bf16", hs, cidx, w, D=wl.D, F=wl.F, E=m + pad, e_begin=0, e_end=m,
                               gate_up_master=gm, down_master=dm)
            t_fwd = time.perf_counter() - t1
            total = t_route + t_fwd
            if total >= target_s or n >= wl.T:
                return {"value": n / total, "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(),
                        "kind": "oracle",
                        "sample": f"first {n} of {wl.T} tokens of the workload, route + forward, "
                                  f"{m} touched experts, {total:.1f} s"}
            n = min(wl.T, max(n * 2, int(n * target_s / max(total, 1e-3)) + 1))
            continue
        gu = {"codes": [], "scales": [], "tensor_scale": []}
        dn = {"codes": [], "scales": [], "tensor_scale": []}
        for e in used:
            e = int(e)
            if e not in quantised:
                quantised[e] = (oracle.quantize_weights(wl.fmt, wl.gate_up_master(e)),
                                oracle.quantize_weights(wl.fmt, wl.down_master(e)))
            for d, q in zip((gu, dn), quantised[e]):
                for key in d:
                    d[key].append(q[key])
        cat = lambda d: {k_: (None if v[0] is None else np.concatenate(v)) for k_, v in d.items()}
        gu, dn = cat(gu), cat(dn)
        pad = max(1, wl.k - m)  # all-zero experts after the m touched ones (the oracle needs E >= top_k)
        t1 = time.perf_counter()
        oracle.moe_forward(wl.fmt, hs, cidx, w, D=wl.D, F=wl.F, E=m + pad, e_begin=0, e_end=m,
                           gate_up=_pad_experts(gu, pad), down=_pad_experts(dn, pad))
        t_fwd = time.perf_counter() - t1
        total = t_route + t_fwd
        if total >= target_s or n >= wl.T:
            return {"value": n / total, "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(),
                    "kind": "oracle",
                    "sample": f"first {n} of {wl.T} tokens of the workload, route + forward, "
                              f"{m} touched experts, {total:.1f} s"}
        n = min(wl.T, max(n * 2, int(n * target_s / max(total, 1e-3)) + 1))


def _pad_experts(d, count):
    """Append `count` all-zero experts (the non-local slot target of the compacted table)."""
    out = {}
    for k_, v in d.items():
        if v is None:
            out[k_] = None
            continue
        pad = np.zeros((count,) + v.shape[1:], v.dtype)
        if k_ == "tensor_scale":  # [E] NVFP4, [E][N] FP8 channel scales
            pad = np.ones((count,) + v.shape[1:], v.dtype)
        out[k_] = np.concatenate([v, pad])
    return out


def run_workload(moe, torch, wl, args, dev):
    """Times one workload: warm-up, then args.steps steps (eager, or one HIP graph replayed per
    step with --graph). Returns its JSON fields."""
    T, D, F, E, k = wl.T, wl.D, wl.F, wl.E, wl.k
    print(f"[bench] workload {wl.index} {wl.name}: T={T} D={D} F={F} E={E} local=[{wl.e_begin},{wl.local_end})",
          file=sys.stderr, flush=True)

    h = wl.hidden()
    wr = wl.router_weight()
    bias = wl.router_bias()
    d_h = torch.from_numpy(h.view(np.int16)).to(dev)
    d_wr = torch.from_numpy(wr.view(np.int16)).to(dev)
    d_bias = None if bias is None else torch.from_numpy(bias).to(dev)
    t0 = time.perf_counter()
    gu, dn = make_weights(moe, torch, wl, dev)
    print(f"[bench] packed weights ready in {time.perf_counter() - t0:.1f} s "
          f"({(gu.nbytes() + dn.nbytes()) / 1e9:.2f} GB)", file=sys.stderr, flush=True)

    layer = moe.Layer(wl.fmt, T, D, F, E, gu, dn, top_k=k, e_begin=wl.e_begin, e_end=wl.local_end)
    plan = layer.plan()  # the kernels moe_forward dispatches (its own plan)
    out = torch.empty((T, D), dtype=torch.float32, device=dev)
    nv = wl.fmt == "nvfp4"
    mx4 = wl.fmt == "mxfp4"

    route_ws = moe.route_workspace(T, D, E, dev)

    def step(events=None):
        idx, w, _, amax = moe.route(d_h, d_wr, k, d_bias, want_amax=nv, workspace=route_ws)
        layer.forward(d_h, idx, w, out=out, h_amax=amax, events=events)
        return idx

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = HipEvents(K * moe.N_EVENTS)
    per_step = [ctypes.cast(ctypes.addressof(ev.arr) + i * moe.N_EVENTS * ctypes.sizeof(ctypes.c_void_p),
                            ctypes.c_void_p) for i in range(K)]
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        idx = step(per_step[i])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    eager_ms_step = total_ms / K
    base = lambda i: i * moe.N_EVENTS
    gate_up_all = [ev.ms(base(i) + 1, base(i) + 2) for i in range(K)]
    fwd_all = [ev.ms(base(i) + 0, base(i) + 5) for i in range(K)]
    gate_up_ms = float(np.mean(gate_up_all))
    down_ms = float(np.mean([ev.ms(base(i) + 3, base(i) + 4) for i in range(K)]))
    fwd_ms = float(np.mean(fwd_all))
    launch = "eager"
    if args.graph:
        # the same step (route + forward, same buffers) captured once as a HIP graph and
        # replayed: the kernels are identical, only the per-launch host and queue gaps go
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            g_idx = step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(K):
            graph.replay()
        stop.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(stop)
        idx = g_idx
        launch = "hip graph per step"
    ms_step = total_ms / K
    ev.close()

    # algorithmic bytes and flops of the dominant kernel (the gate_up GEMM)
    idx_h = idx.cpu().numpy()
    local = (idx_h >= wl.e_begin) & (idx_h < wl.local_end)
    S = int(local.sum())
    touched = int(len(np.unique(idx_h[local])))
    gu_b = packed_bytes_per_expert(wl.fmt, 2 * F, D)
    dn_b = packed_bytes_per_expert(wl.fmt, D, F)
    code_b = {"nvfp4": lambda c: c // 2 + c // 16, "mxfp4": lambda c: c // 2 + c // 32,
              "mxfp8": lambda c: c + c // 32, "w4a16": lambda c: 2 * c, "bf16": lambda c: 2 * c,
              "fp8": lambda c: c + 4}[wl.fmt]
    act_b = lambda rows, cols: rows * code_b(cols)
    gate_up_bytes = touched * gu_b + act_b(T, D) + act_b(S, F)
    gate_up_flops = 4.0 * S * F * D
    layer_bytes = touched * (gu_b + dn_b) + E * D * 2 + T * D * 2 + T * D * 4
    # the contraction's own peak: NVFP4 runs the f16 MFMA on exactly expanded values, W4A16
    # and bf16 experts the bf16 MFMA, MXFP4 the scaled FP4 MFMA, MXFP8 and FP8 the scaled FP8
    # MFMA (MXFP8 with exact sums: the bf16 MFMA); the format's scaled-MFMA peak is reported
    # beside it
    kern = plan["gate_up_kernel"]
    native8 = wl.fmt in ("mxfp8", "fp8") and kern in ("mx_gemm_kernel", "fp8_wide_gemm_kernel")
    mfma_peak = MFMA_PEAK_TFLOPS["fp4" if mx4 else ("f16" if nv else ("fp8" if native8 else "bf16"))]
    format_peak = MFMA_PEAK_TFLOPS["fp4" if nv or mx4 else ("bf16" if wl.fmt in ("w4a16", "bf16") else "fp8")]
    decode = 6.0 * S * D * F / max(layer_bytes, 1) < mfma_peak / HBM_PEAK_GBS * 1e3  # below the ridge
    if decode:
        achieved = gate_up_bytes / (gate_up_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = gate_up_flops / (gate_up_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(achieved / mfma_peak, 4), "traffic": None,
                "format_scaled_mfma": {"peak": format_peak, "frac": round(achieved / format_peak, 4)}}
    # the attainable roofline of the launch: min(peak, arithmetic intensity x HBM peak)
    if roof["bound"] == "mfma":
        att = min(mfma_peak, gate_up_flops / gate_up_bytes * HBM_PEAK_GBS / 1e3)
        roof["attainable"] = {"peak": round(att, 1), "frac": round(achieved / att, 4)}
    roof["traffic"] = profiled_traffic(wl.name, kern)
    roof["kernel"] = f"{kern} (gate_up)"
    roof["kernel_source_sha256"] = kernel_source_hash(kern)
    roof["per_launch"] = {"bytes": gate_up_bytes, "flops": gate_up_flops, "ms": round(gate_up_ms, 4)}

    print(f"[bench] {wl.name}: {ms_step:.3f} ms/step ({launch}; eager {eager_ms_step:.3f}) (forward {fwd_ms:.3f} ms: "
          f"gate_up {gate_up_ms:.3f} ms, down {down_ms:.3f} ms); S={S}, {touched} experts touched, layer "
          f"{layer_bytes / 1e9:.3f} GB -> {layer_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s whole-step; "
          f"{plan['gate_up_kernel']} / {plan['down_kernel']}", file=sys.stderr, flush=True)

    if args.calib_copy_mb:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the counters
        n = args.calib_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        del src, dst

    del layer, gu, dn, out, route_ws, d_h, d_wr, d_bias
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, h, wr, bias, args.cpu_target_s)
        print(f"[bench] {wl.name} cpu baseline: {cpu}", file=sys.stderr, flush=True)

    return {
        "value": round(T * K / (total_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms_step, 4),
        "dtype": DTYPES[wl.fmt] if wl.fmt != "mxfp8" or native8 else "bf16 (exact MXFP8 values), fp32 accumulate",
        "config": {"workload": wl.name, "launch": launch, "tokens": T, "d_model": D, "d_ff": F, "experts": E,
                   "top_k": k, "format": wl.fmt, "local_experts": [wl.e_begin, wl.local_end],
                   "experts_touched": touched, "slots": S, "layer_bytes": layer_bytes,
                   "layer_GBps": round(layer_bytes / (ms_step * 1e-3) / 1e9, 1),
                   "kernels": {"gate_up": plan["gate_up_kernel"], "down": plan["down_kernel"]},
                   "stage_ms": {"forward": round(fwd_ms, 4), "gate_up": round(gate_up_ms, 4),
                                "down": round(down_ms, 4),
                                "forward_median": round(float(np.median(fwd_all)), 4),
                                "forward_min": round(float(np.min(fwd_all)), 4),
                                "gate_up_median": round(float(np.median(gate_up_all)), 4),
                                "gate_up_min": round(float(np.min(gate_up_all)), 4)}},
        "roofline": roof,
        "cpu_baseline": cpu,
    }


# the layer's five configurations (bench workloads 0-4); decode-nvfp4 is the headline
DEFAULT_WORKLOADS = [0, 1, 2, 3, 4]
HEADLINE = 1


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=None,
                    help="run one of the thirteen synthetic workloads alone (default: the five configurations)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time one captured HIP graph per step, replayed (default: eager launches; on MI355X "
                         "the two measured the same)")
    ap.add_argument("--cpu-target-s", type=float, default=None,
                    help="seconds of oracle work per workload (default: 10 for one workload, 6 each for the five)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the layer is built for one "
              "GPU's expert share (moe_forward takes a local expert range; N ranks would each run the "
              "same router, compute their experts' slots and sum the fp32 partial outputs with one "
              "all-reduce).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_scaled_moe_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    workloads = DEFAULT_WORKLOADS if args.workload is None else [args.workload]
    if args.cpu_target_s is None:
        args.cpu_target_s = 10.0 if len(workloads) == 1 else 6.0
    results = [run_workload(moe, torch, synth.WORKLOADS[i], args, dev) for i in workloads]
    head = results[workloads.index(HEADLINE)] if HEADLINE in workloads else results[0]

    line = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
        "config": head["config"], "roofline": head["roofline"], "cpu_baseline": head["cpu_baseline"],
    }
    if len(results) > 1:
        line["configs"] = [{"workload": r["config"]["workload"], "value": r["value"], "unit": r["unit"],
                            "ms_per_step": r["ms_per_step"], "dtype": r["dtype"], "config": r["config"],
                            "roofline": r["roofline"], "cpu_baseline": r["cpu_baseline"]} for r in results]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
