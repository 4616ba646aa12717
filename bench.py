#!/usr/bin/env python3
"""Throughput of the transposed-convolution forward on one MI355X.

A step is one call of the whole hot path (one convt_forward or
convt_forward_add_hswish launch) over one batch of seeded synthetic input
already resident in HBM.  W untimed warm-up steps, then exactly K timed steps
between two device synchronisations; HIP events on the stream the kernel is
launched on (torch's current stream, which the binding passes to the library)
time the region and every launch.

Prints ONE JSON line.  The headline (`value`) is the long-sequence 1D layer
(N=16, 32->64 channels, L=131072, K=3, stride 2, padding 1, dilation 2):
  value         algorithmic GB/s (x + w + bias + y [+ add_input], each once)
                over the K back-to-back steps
  roofline      the kernel's achieved rate against the MI355X peak that bounds
                it (average launch time over the timed region), with the same
                figure under the cache-flushed protocol (a 512 MB write and a
                512 MB read of other buffers before every launch, so no launch
                finds its inputs in, or leaves its outputs to, the 256 MB
                last-level cache of the one before) and against the measured
                ceilings below
  configs       the same measurement for every workload (the tiny, long 1D,
                grouped 3D, fused 3D and channel-heavy 3D layers), each with
                its roofline, flushed figure, counter traffic and CPU baseline
  calibration   measured ceilings on this GPU: copy, fill and read bandwidth,
                the long 1D layer's byte mix as two flat streams and in the
                layer's own access pattern (no arithmetic), and a register-only
                fp32 MFMA chain
  cpu_baseline  the fp64 CPU oracle, untuned, on a bounded sample of the same
                workload, in the same unit (with the host CPU model, its
                os.cpu_count() and a single-thread figure for the small layers)

--op backward_data / backward_weight time the input gradient (dy and w in, dx
out) or the weight and bias gradients (x and dy in, dw and db out) instead.
--memory-floor runs only the calibration kernels (for a profiler run);
--copy-calibration times a plain 1 GiB copy (used to scale the HBM byte
counters of a profiler run).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import transposed_convolution_forward_amd as T  # noqa: E402
from transposed_convolution_forward_amd import synthetic as S  # noqa: E402

PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 (matrix and vector)
KERNEL_NAMES = {"generic": "k_generic", "stream1d": "k_stream1d", "igemm3d": "k_igemm3d"}
FLUSH_BYTES = 512 << 20     # each of the write and the read before a flushed launch
CONFIG_KEYS = {S.TINY_1D.name: "cfg1_tiny_1d", S.LONG_1D.name: "cfg2_long_1d",
               S.GROUPED_3D.name: "cfg3_grouped_3d", S.FUSED_3D.name: "cfg4_fused_3d",
               S.HEAVY_3D.name: "cfg5_channel_heavy_3d"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def out_size(wl):
    return tuple((wl.in_size[a] - 1) * wl.stride[a] - 2 * wl.pad[a] +
                 wl.dilation[a] * (wl.K[a] - 1) + wl.out_pad[a] + 1 for a in range(wl.ndim))


def algorithmic_bytes(wl, N=None):
    N = wl.N if N is None else N
    ys = N * wl.C_out * int(np.prod(out_size(wl)))
    b = N * wl.C_in * int(np.prod(wl.in_size)) + int(np.prod(wl.w_shape())) + ys
    if wl.bias:
        b += wl.C_out
    if wl.fused:
        b += ys
    return 4 * b


def algorithmic_bytes_backward(wl, N=None):
    """Input gradient: dy + w + dx, each once."""
    N = wl.N if N is None else N
    return 4 * (N * wl.C_out * int(np.prod(out_size(wl))) + int(np.prod(wl.w_shape())) +
                N * wl.C_in * int(np.prod(wl.in_size)))


def algorithmic_bytes_weight(wl, N=None):
    """Weight and bias gradients: x + dy + dw + db, each once."""
    N = wl.N if N is None else N
    return 4 * (N * wl.C_in * int(np.prod(wl.in_size)) + N * wl.C_out * int(np.prod(out_size(wl))) +
                int(np.prod(wl.w_shape())) + wl.C_out)


def op_bytes(wl, op, N=None):
    return {"forward": algorithmic_bytes, "backward_data": algorithmic_bytes_backward,
            "backward_weight": algorithmic_bytes_weight}[op](wl, N)


def valid_macs(wl, N=None):
    """N*C_in*(C_out/g)*prod_a #{(i,k): 0 <= i*s - p + k*d < L_out} (taps that
    land inside the output; the dense work the phase split skips is not
    counted)."""
    N = wl.N if N is None else N
    P = 1
    for a, Lo in enumerate(out_size(wl)):
        i = np.arange(wl.in_size[a])[:, None]
        k = np.arange(wl.K[a])[None, :]
        o = i * wl.stride[a] - wl.pad[a] + k * wl.dilation[a]
        P *= int(np.count_nonzero((o >= 0) & (o < Lo)))
    return N * wl.C_in * (wl.C_out // wl.groups) * P


# The source file each kernel is built from; with the headers every kernel
# includes, it decides whether a stored counter record still describes the
# kernel that runs.
KERNEL_SOURCES = {"k_stream1d": "stream1d.hip", "k_stream1d_nlc": "stream1d.hip", "k_igemm3d": "igemm3d.hip",
                  "k_igemm3d_wide": "igemm3d.hip", "k_generic_nxc": "generic.hip",
                  "k_generic": "generic.hip", "k_generic_phase": "generic.hip", "k_generic_rows": "generic.hip",
                  "k_generic_pairs": "generic.hip", "k_generic_wpair": "wpair.hip", "k_backward_data": "backward.hip",
                  "k_backward_data_mfma": "backward.hip", "k_backward_data_mfma_row": "backward.hip",
                  "k_backward_data_wpair": "backward.hip", "k_backward_data_stage": "backward.hip",
                  "k_backward_weight": "wgrad.hip", "k_backward_weight_lds": "wgrad.hip",
                  "k_backward_weight_row": "wgrad.hip", "k_backward_weight_shift": "wgrad.hip",
                  "k_backward_weight_shift_rows": "wgrad.hip", "k_backward_weight_stage": "wgrad.hip",
                  "k_backward_bias": "wgrad.hip"}
SHARED_SOURCES = ("convt_internal.h", "epilogue.hpp")


def source_sha(kernel=None):
    """Hash of the kernel's own source and the shared headers (of every
    kernel source when kernel is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transposed_convolution_forward_amd", "csrc")
    if kernel is None:
        files = sorted(f for f in glob.glob(os.path.join(csrc, "*")) if f.endswith((".hip", ".cpp", ".h", ".hpp")))
    else:
        files = [os.path.join(csrc, f) for f in (KERNEL_SOURCES.get(kernel, "generic.hip"),) + SHARED_SOURCES]
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_key(wl_name, layout="channels_first"):
    return wl_name if layout == "channels_first" else f"{wl_name}_{layout}"


def traffic_for(wl_name, kernel, layout="channels_first"):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(traffic_key(wl_name, layout))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel or rec.get("source_sha") != source_sha(kernel):
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def host_cpu():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def _oracle_run(orc, wl, inp, op, n_s, threads, layout=0):
    shape = dict(ndim=wl.ndim, N=n_s, C_in=wl.C_in, C_out=wl.C_out, groups=wl.groups,
                 in_size=wl.in_size, K=wl.K, stride=wl.stride, pad=wl.pad, out_pad=wl.out_pad,
                 dilation=wl.dilation, nthreads=threads)
    if layout:
        shape["layout"] = layout
    t0 = time.perf_counter()
    if op == "backward_data":
        orc.backward_data(dy=np.ascontiguousarray(inp["dy"][:n_s]), w=inp["w"], **shape)
    elif op == "backward_weight":
        orc.backward_weight(x=np.ascontiguousarray(inp["x"][:n_s]), dy=np.ascontiguousarray(inp["dy"][:n_s]),
                            **shape)
    else:
        orc.forward(x=np.ascontiguousarray(inp["x"][:n_s]), w=inp["w"], bias=inp["bias"],
                    add=None if inp["add"] is None else np.ascontiguousarray(inp["add"][:n_s]), **shape)
    return time.perf_counter() - t0


def cpu_baseline(wl, inp, op="forward", single_thread=False, layout=0):
    """The oracle (as it stands) on the first n_s batch samples, with as many
    threads as it can use there (it splits the work by (sample, group), or by
    input channel for the weight gradient), at most 16; optionally also with
    one thread on one sample."""
    import oracle
    orc = oracle.get()
    cores = min(16, os.cpu_count() or 1)
    n_s = max(1, min(wl.N, cores // max(1, wl.groups)))
    threads = min(cores, wl.C_in) if op == "backward_weight" else min(cores, n_s * wl.groups)
    dt = _oracle_run(orc, wl, inp, op, n_s, threads, layout)
    nbytes = op_bytes(wl, op, n_s)
    kind = dict(backward_data="adjoint", backward_weight="weight-gradient").get(op, "scatter")
    res = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"first {n_s} of {wl.N} batch samples (all channels and positions), "
                     f"{dt:.2f} s wall; fp64 {kind} loop, {threads} threads",
           "valid_mac_gflops": 2 * valid_macs(wl, n_s) / dt / 1e9, "wall_s": round(dt, 3)}
    res.update(host_cpu())
    if single_thread:
        dt1 = _oracle_run(orc, wl, inp, op, 1, 1, layout)
        res["single_thread"] = {"value": op_bytes(wl, op, 1) / dt1 / 1e9, "unit": "GB/s",
                                "sample": f"first 1 of {wl.N} batch samples, 1 thread",
                                "wall_s": round(dt1, 3)}
    return res


# --- calibration kernels (libconvt_calib.so, measurement only) ------------
_calib = None


def calib_lib():
    import ctypes
    global _calib
    if _calib is None:
        path = os.path.join(ROOT, "transposed_convolution_forward_amd", "libconvt_calib.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m transposed_convolution_forward_amd.build`")
        L = ctypes.CDLL(path)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.convt_calib_fill.argtypes = [vp, i64, ci, vp]
        L.convt_calib_read.argtypes = [vp, i64, ci, vp, vp]
        L.convt_calib_copy.argtypes = [vp, vp, i64, ci, vp]
        L.convt_calib_mixed.argtypes = [vp, i64, vp, i64, ci, vp]
        L.convt_calib_ncl_1d.argtypes = [vp, vp, i64, ci, ci, ci, ci, vp]
        L.convt_calib_mfma_f32.argtypes = [ci, ci, ci, vp, vp]
        for f in ("fill", "read", "copy", "mixed", "ncl_1d", "mfma_f32"):
            getattr(L, "convt_calib_" + f).restype = ctypes.c_int
        _calib = L
    return _calib


def _stream():
    import torch
    return torch.cuda.current_stream()


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: HIP error {rc}")


class Flusher:
    """Before a flushed launch: a 512 MB write (fill) and a 512 MB read of
    two other buffers, so that the 256 MB last-level cache holds neither the
    launch's inputs nor dirty lines of earlier work."""

    def __init__(self):
        import torch
        self.w = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.r = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.out = torch.empty(8192, dtype=torch.float32, device="cuda")

    def __call__(self):
        L, s = calib_lib(), _stream().cuda_stream
        _check(L.convt_calib_fill(self.w.data_ptr(), FLUSH_BYTES // 16, 1024, s), "flush fill")
        _check(L.convt_calib_read(self.r.data_ptr(), FLUSH_BYTES // 16, 1024, self.out.data_ptr(), s), "flush read")


def time_launches(fn, n, before=None):
    """Per-launch milliseconds of n launches of fn on the current stream (HIP
    events on that stream), each optionally preceded by before() outside its
    events; and the whole region's milliseconds."""
    import torch
    stream = _stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a0.record(stream)
    for i in range(n):
        if before is not None:
            before()
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    a1.record(stream)
    torch.cuda.synchronize()
    return np.array([x.elapsed_time(y) for x, y in ev]), a0.elapsed_time(a1)


def calibration(reps=10):
    """Measured ceilings: copy / fill / read of 1 GiB, the long 1D layer's byte
    mix (x read 268 MB, y written 1.07 GB) as two flat streams and in the
    layer's own pattern, and a register-only fp32 MFMA chain."""
    import torch
    L, s = calib_lib(), _stream().cuda_stream
    n4 = (1 << 30) // 16
    a = torch.ones(n4 * 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = torch.empty(8192, dtype=torch.float32, device="cuda")
    res = {}

    def med(fn):
        for _ in range(3):
            fn()
        t, _ = time_launches(fn, reps)
        return float(np.median(t))

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sweep = (2 * cus, 4 * cus, 8 * cus)  # workgroups; the best of the sweep is the ceiling

    def best(fn, nbytes):
        per = {bl: nbytes / (med(lambda: fn(bl)) * 1e-3) / 1e9 for bl in sweep}
        bl = max(per, key=per.get)
        return round(per[bl], 1), bl

    res["copy_gbs"], res["copy_blocks"] = best(
        lambda bl: _check(L.convt_calib_copy(a.data_ptr(), b.data_ptr(), n4, bl, s), "copy"), 2 * 16 * n4)
    res["fill_gbs"], res["fill_blocks"] = best(
        lambda bl: _check(L.convt_calib_fill(b.data_ptr(), n4, bl, s), "fill"), 16 * n4)
    res["read_gbs"], res["read_blocks"] = best(
        lambda bl: _check(L.convt_calib_read(a.data_ptr(), n4, bl, out.data_ptr(), s), "read"), 16 * n4)
    del a, b
    wl = S.LONG_1D
    Lo = out_size(wl)[0]
    x = torch.ones((wl.N, wl.C_in, wl.in_size[0]), dtype=torch.float32, device="cuda")
    y = torch.empty((wl.N, wl.C_out, Lo), dtype=torch.float32, device="cuda")
    nbytes = 4 * (x.numel() + y.numel())
    blocks = torch.cuda.get_device_properties(0).multi_processor_count * 3
    t = med(lambda: _check(L.convt_calib_mixed(x.data_ptr(), x.numel() // 4, y.data_ptr(), y.numel() // 4,
                                               blocks, s), "mixed"))
    res["long_1d_flat_streams"] = {"ms": round(t, 5), "gbs": round(nbytes / (t * 1e-3) / 1e9, 1),
                                   "bytes": nbytes, "what": "x read and y written as two flat streams, "
                                   "items of 8 KB read + 32 KB written, same workgroup count as stream1d"}
    ncl = lambda: _check(L.convt_calib_ncl_1d(x.data_ptr(), y.data_ptr(), wl.N, wl.in_size[0], Lo, wl.pad[0],
                                              blocks, s), "ncl_1d")
    t = med(ncl)
    # the same after the flush the flushed launches get (512 MB written, 512 MB read)
    flusher = Flusher()
    tf, _ = time_launches(ncl, reps, before=flusher)
    del flusher
    tf = float(np.median(tf))
    res["long_1d_layer_pattern"] = {"ms": round(t, 5), "gbs": round(nbytes / (t * 1e-3) / 1e9, 1),
                                    "ms_flushed": round(tf, 5), "gbs_flushed": round(nbytes / (tf * 1e-3) / 1e9, 1),
                                    "bytes": nbytes, "what": "the layer's per-item 32 x 68 x tile read and "
                                    "64 row segments of 128 floats written from 128-byte line boundaries "
                                    "(non-temporal), no arithmetic; back to back and after a cache flush"}
    del x, y
    iters = 4096
    per = {}
    for wps in (1, 2):
        t = med(lambda: _check(L.convt_calib_mfma_f32(cus, wps, iters, out.data_ptr(), s), "mfma"))
        per[wps] = cus * 4 * wps * iters * 8 * 2 * 16 * 16 * 4 / (t * 1e-3) / 1e12
    wps = max(per, key=per.get)
    res["mfma_f32_tflops"] = round(per[wps], 2)
    res["mfma_by_waves_per_simd"] = {str(k): round(v, 2) for k, v in per.items()}
    res["mfma_what"] = "v_mfma_f32_16x16x4_f32 register-only, 8 independent accumulators per wave"
    res["hbm_gbs"] = max(res["copy_gbs"], res["fill_gbs"], res["read_gbs"], res["long_1d_flat_streams"]["gbs"],
                         res["long_1d_layer_pattern"]["gbs"])
    res["hbm_what"] = "the best of the bandwidth figures above"
    return res


def copy_calibration(steps):
    import torch
    n = 1 << 28  # 1 GiB of float32
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": steps}))


def kernel_of(plan, op, path):
    text = T.convt_plan_describe(plan)
    pat = {"backward_data": r"input gradient: kernel=(\S+)", "backward_weight": r"weight gradient: kernel=(\S+)"}
    m = re.search(pat.get(op, r"kernel=(\S+)"), text)
    return m.group(1) if m else KERNEL_NAMES.get(path, path)


def measure(wl, op, steps, warmup, path="auto", flushed=20, flusher=None, cpu=True, single_thread=False,
            layout="channels_first"):
    """One workload: warm-up, K back-to-back timed launches, then `flushed`
    launches each after the cache flush; roofline figures and the CPU
    baseline.  Channels last takes the seeded channels-first draws with the
    channel axis moved last.  Returns (record, ms_per_step, timed wall
    seconds)."""
    import torch
    log(f"workload {wl.name} ({op}, {layout}): generating seeded inputs")
    bwd, wgr = op == "backward_data", op == "backward_weight"
    inp = S.make_inputs(wl, 0, (wl.N, wl.C_out) + out_size(wl))
    if bwd:
        inp = {"dy": S.make_grad_output(wl, 0, (wl.N, wl.C_out) + out_size(wl)), "w": inp["w"]}
    elif wgr:
        inp = {"dy": S.make_grad_output(wl, 0, (wl.N, wl.C_out) + out_size(wl)), "x": inp["x"]}
    if layout == "channels_last":
        for k in ("x", "add"):
            if inp.get(k) is not None:
                inp[k] = np.ascontiguousarray(np.moveaxis(inp[k], 1, -1))
    dev = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inp.items()}
    plan = T.plan_for(wl, layout)
    if path != "auto":
        T.convt_plan_set_path(plan, path)
    path = T.convt_plan_get_path(plan)
    y = torch.empty(plan.x_shape() if bwd else plan.w_shape() if wgr else plan.y_shape(), dtype=torch.float32,
                    device="cuda")
    db = torch.empty((wl.C_out,), dtype=torch.float32, device="cuda")

    def step():
        if bwd:
            T.convt_backward_data(plan, dev["dy"], dev["w"], dx=y)
        elif wgr:
            T.convt_backward_weight(plan, dev["x"], dev["dy"], dw=y, db=db)
        elif wl.fused:
            T.convt_forward_add_hswish(plan, dev["x"], dev["w"], dev["bias"], dev["add"], y=y)
        else:
            T.convt_forward(plan, dev["x"], dev["w"], dev["bias"], y=y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"path {path}: warm-up done, timing {steps} steps")
    wall0 = time.perf_counter()
    launches, total_ms = time_launches(step, steps)
    wall = time.perf_counter() - wall0
    ms_per_step = total_ms / steps
    ms_launch = float(launches.mean())
    cold = None
    if flushed > 0:
        flusher = flusher or Flusher()
        cold, _ = time_launches(step, flushed, before=flusher)

    nbytes = op_bytes(wl, op)
    flops = 2 * valid_macs(wl)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_fp32 = flops / (PEAK_FP32_TFLOPS * 1e12)
    kernel = kernel_of(plan, op, path)
    stats = lambda a: {"median": round(float(np.median(a)), 5), "min": round(float(a.min()), 5),
                       "max": round(float(a.max()), 5)}
    if t_hbm >= t_fp32:
        rate = lambda ms: nbytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(rate(ms_launch), 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(rate(ms_launch) / PEAK_HBM_GBS, 4)}
    else:
        rate = lambda ms: flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(rate(ms_launch), 2), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(rate(ms_launch) / PEAK_FP32_TFLOPS, 4)}
    roof["traffic"] = traffic_for(wl.name, kernel, layout) if op == "forward" else None
    roof["kernel"] = kernel
    roof["launch_ms"] = round(ms_launch, 5)
    roof["launch_ms_stats"] = stats(launches)
    if cold is not None:
        cold_ms = float(np.median(cold))
        roof["flushed"] = dict(stats(cold), launches=int(flushed),
                               achieved=round(rate(cold_ms), 2 if roof["bound"] == "mfma" else 1),
                               frac=round(rate(cold_ms) / roof["peak"], 4))
    rec = {"workload": wl.name, "op": op, "layout": layout, "path": path, "kernel": kernel,
           "ms_per_step": round(ms_per_step, 5), "gbs": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
           "valid_mac_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
           "hbm_frac": round(t_hbm / (ms_per_step * 1e-3), 4), "fp32_frac": round(t_fp32 / (ms_per_step * 1e-3), 4),
           "algorithmic_bytes": nbytes, "valid_macs": flops // 2, "roofline": roof}
    del dev, y, db
    torch.cuda.empty_cache()
    if cpu:
        log(f"timing the CPU oracle on a bounded sample of {wl.name}")
        rec["cpu_baseline"] = cpu_baseline(wl, inp, op=op, single_thread=single_thread,
                                           layout=1 if layout == "channels_last" else 0)
    return rec, ms_per_step, wall


def against_measured(rec, cal):
    """The roofline fractions against the measured ceilings: the best
    measured HBM stream rate for an HBM-bound launch, the MFMA chain for an
    MFMA-bound one."""
    roof = rec["roofline"]
    ms = roof["launch_ms"]
    fl = roof.get("flushed", {}).get("median")
    if roof["bound"] == "hbm":
        peak = cal["hbm_gbs"]
        rate = lambda m: rec["algorithmic_bytes"] / (m * 1e-3) / 1e9
        out = {"peak": peak, "unit": "GB/s", "what": "best measured HBM stream rate (calibration.hbm_gbs)"}
    else:
        peak = cal["mfma_f32_tflops"]
        rate = lambda m: 2 * rec["valid_macs"] / (m * 1e-3) / 1e12
        out = {"peak": peak, "unit": "TFLOP/s", "what": "measured fp32 MFMA chain"}
    out["frac"] = round(rate(ms) / peak, 4)
    if fl:
        out["frac_flushed"] = round(rate(fl) / peak, 4)
    roof["vs_measured"] = out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=S.LONG_1D.name, choices=sorted(S.BY_NAME))
    ap.add_argument("--path", default="auto", choices=sorted(T.PATHS))
    ap.add_argument("--layout", default="channels_first", choices=sorted(T.LAYOUTS),
                    help="layout of x, y and add_input for the headline workload")
    ap.add_argument("--op", default="forward", choices=["forward", "backward_data", "backward_weight"],
                    help="forward (the hot path, default), the input gradient, or the weight and bias gradients")
    ap.add_argument("--flushed", type=int, default=20, help="cache-flushed launches per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the calibration kernels (e.g. under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--memory-floor", action="store_true",
                    help="run only the calibration kernels and print their figures")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "forward needs no collective and shards by batch with no exchange, but no "
              "multi-GPU run is implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.memory_floor:
        log("calibration kernels only")
        print(json.dumps({"calibration": calibration()}), flush=True)
        return

    wl = S.BY_NAME[args.workload]
    flusher = Flusher() if args.flushed > 0 else None
    head, ms_per_step, wall = measure(wl, args.op, args.steps, args.warmup, args.path, args.flushed, flusher,
                                      cpu=not args.no_cpu_baseline, single_thread=wl.name != S.HEAVY_3D.name and
                                      wl.name != S.FUSED_3D.name, layout=args.layout)
    configs = {}
    if not args.no_configs:
        for other in S.WORKLOADS:
            key = CONFIG_KEYS[other.name]
            if other.name == wl.name and args.layout == "channels_first":
                configs[key] = head
                continue
            rec, _, _ = measure(other, args.op, args.steps, args.warmup, "auto", args.flushed, flusher,
                                cpu=not args.no_cpu_baseline,
                                single_thread=other.name in (S.TINY_1D.name, S.LONG_1D.name, S.GROUPED_3D.name))
            configs[key] = rec
        if args.op == "forward":
            # the channels-last layout of the long 1D, fused 3D and channel-heavy 3D layers
            for other in (S.LONG_1D, S.FUSED_3D, S.HEAVY_3D):
                rec, _, _ = measure(other, args.op, args.steps, args.warmup, "auto", args.flushed, flusher,
                                    cpu=not args.no_cpu_baseline, layout="channels_last")
                configs[CONFIG_KEYS[other.name] + "_channels_last"] = rec
    del flusher
    torch.cuda.empty_cache()
    cal = None
    if not args.no_calibration:
        log("calibration kernels")
        cal = calibration()
        for rec in [head] + list(configs.values()):
            against_measured(rec, cal)
    if cal is not None and wl.name == S.LONG_1D.name and args.op == "forward":
        floor = cal["long_1d_layer_pattern"]["ms"]
        floor_fl = cal["long_1d_layer_pattern"]["ms_flushed"]
        head["roofline"]["vs_memory_floor"] = {
            "floor_ms": floor, "floor_ms_flushed": floor_fl,
            "floor_what": "the layer's own memory pattern without arithmetic (back to back; after a cache flush)",
            "frac": round(floor / head["roofline"]["launch_ms"], 4),
            "frac_flushed": round(floor_fl / head["roofline"]["flushed"]["median"], 4) if "flushed" in head["roofline"]
            else None}

    metric = {"backward_data": "ConvTranspose input-gradient GB/s and valid-MAC TFLOP/s, % of roofline, 1x MI355X",
              "backward_weight": "ConvTranspose weight-gradient GB/s and valid-MAC TFLOP/s, % of roofline, 1x MI355X"
              }.get(args.op, "ConvTranspose fwd GB/s and valid-MAC TFLOP/s, % of roofline, 1x MI355X")
    line = {
        "metric": metric,
        "value": head["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded: x, add ~ N(0,1); w, bias ~ U(+-1/sqrt(fan_in)))",
        "config": {"workload": wl.name, "ndim": wl.ndim, "N": wl.N, "C_in": wl.C_in,
                   "C_out": wl.C_out, "groups": wl.groups, "in_size": list(wl.in_size),
                   "out_size": list(out_size(wl)), "K": list(wl.K), "stride": list(wl.stride),
                   "pad": list(wl.pad), "out_pad": list(wl.out_pad),
                   "dilation": list(wl.dilation), "bias": wl.bias, "fused": wl.fused,
                   "path": head["path"], "op": args.op, "layout": args.layout, "parallelism": "single GPU"},
        "valid_mac_tflops": head["valid_mac_tflops"], "hbm_frac": head["hbm_frac"], "fp32_frac": head["fp32_frac"],
        "algorithmic_bytes": head["algorithmic_bytes"], "valid_macs": head["valid_macs"],
        "timed_wall_s": round(wall, 4), "source_sha": source_sha(),
        "roofline": head["roofline"], "cpu_baseline": head.get("cpu_baseline"),
        "configs": configs,
        "calibration": cal,
        "protocol": {"timed": f"{args.steps} back-to-back launches after {args.warmup} warm-up, HIP events on "
                              "the launch stream; roofline.achieved from their mean",
                     "flushed": f"{args.flushed} launches, each after a {FLUSH_BYTES >> 20} MB write and a "
                                f"{FLUSH_BYTES >> 20} MB read of other buffers (the 256 MB last-level cache "
                                "evicted); median"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
