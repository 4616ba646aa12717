#!/usr/bin/env python3
"""Throughput of the transposed-convolution forward on one MI355X.

A step is one call of the whole hot path (one convt_forward or
convt_forward_add_hswish launch) over one batch of seeded synthetic input
already resident in HBM.  W untimed warm-up steps, then exactly K timed steps
between two device synchronisations; HIP events on the stream the kernel is
launched on (torch's current stream, which the binding passes to the library)
time the region and every launch.

Prints ONE JSON line (the default workload is the long-sequence 1D layer,
N=16, 32->64 channels, L=131072, K=3, stride 2, padding 1, dilation 2):
  value      algorithmic GB/s (x + w + bias + y [+ add_input], each once)
  roofline   the kernel's achieved rate against the MI355X peak that bounds it
  cpu_baseline  the fp64 CPU oracle, untuned, on a bounded sample of the same
             workload, in the same unit.

--op backward_data times the input gradient (convt_backward_data: dy and w in,
dx out) on the same workload instead of the forward; its bytes are dy + w + dx
and its valid MACs those of the forward.  --op backward_weight times the
weight and bias gradients (convt_backward_weight: x and dy in, dw and db out;
bytes x + dy + dw + db, the same valid MACs).

--copy-calibration instead times a plain 1 GiB device copy (used to scale the
HBM byte counters of a profiler run).
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
KERNEL_SOURCES = {"k_stream1d": "stream1d.hip", "k_igemm3d": "igemm3d.hip", "k_igemm3d_wide": "igemm3d.hip",
                  "k_generic": "generic.hip", "k_generic_phase": "generic.hip", "k_generic_rows": "generic.hip",
                  "k_generic_pairs": "generic.hip", "k_backward_data": "backward.hip",
                  "k_backward_data_mfma": "backward.hip", "k_backward_data_mfma_row": "backward.hip",
                  "k_backward_weight": "wgrad.hip",
                  "k_backward_weight_lds": "wgrad.hip", "k_backward_weight_row": "wgrad.hip"}
SHARED_SOURCES = ("convt_internal.h", "epilogue.hpp")


def source_sha(kernel=None):
    """Hash of the kernel's own source and the shared headers (of every
    kernel source when kernel is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transposed_convolution_forward_amd", "csrc")
    if kernel is None:
        files = sorted(f for f in glob.glob(os.path.join(csrc, "*")) if f.endswith((".hip", ".cpp", ".h", ".hpp")))
    else:
        files = [os.path.join(csrc, f) for f in (KERNEL_SOURCES[kernel],) + SHARED_SOURCES]
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(wl_name, kernel):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(wl_name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel or rec.get("source_sha") != source_sha(kernel):
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def cpu_baseline(wl, inp, budget_slabs=None, op="forward"):
    """The oracle (as it stands) on the first n_s batch samples."""
    import oracle
    orc = oracle.get()
    cores = min(16, os.cpu_count() or 1)
    n_s = budget_slabs or max(1, min(wl.N, cores // max(1, wl.groups)))
    threads = min(cores, n_s * wl.groups)
    shape = dict(ndim=wl.ndim, N=n_s, C_in=wl.C_in, C_out=wl.C_out, groups=wl.groups,
                 in_size=wl.in_size, K=wl.K, stride=wl.stride, pad=wl.pad, out_pad=wl.out_pad,
                 dilation=wl.dilation, nthreads=threads)
    t0 = time.perf_counter()
    if op == "backward_data":
        orc.backward_data(dy=np.ascontiguousarray(inp["dy"][:n_s]), w=inp["w"], **shape)
        nbytes = algorithmic_bytes_backward(wl, n_s)
    elif op == "backward_weight":
        shape["nthreads"] = min(cores, wl.C_in)
        threads = shape["nthreads"]
        orc.backward_weight(x=np.ascontiguousarray(inp["x"][:n_s]), dy=np.ascontiguousarray(inp["dy"][:n_s]),
                            **shape)
        nbytes = algorithmic_bytes_weight(wl, n_s)
    else:
        orc.forward(x=np.ascontiguousarray(inp["x"][:n_s]), w=inp["w"], bias=inp["bias"],
                    add=None if inp["add"] is None else np.ascontiguousarray(inp["add"][:n_s]), **shape)
        nbytes = algorithmic_bytes(wl, n_s)
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {n_s} of {wl.N} batch samples (all channels and positions), "
                      f"{dt:.2f} s wall; fp64 {dict(backward_data='adjoint', backward_weight='weight-gradient').get(op, 'scatter')} loop, "
                      f"{threads} threads",
            "valid_mac_gflops": 2 * valid_macs(wl, n_s) / dt / 1e9}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=S.LONG_1D.name, choices=sorted(S.BY_NAME))
    ap.add_argument("--path", default="auto", choices=sorted(T.PATHS))
    ap.add_argument("--op", default="forward", choices=["forward", "backward_data", "backward_weight"],
                    help="forward (the hot path, default), the input gradient, or the weight and bias gradients")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
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

    wl = S.BY_NAME[args.workload]
    print(f"[bench] workload {wl.name}: generating seeded inputs", file=sys.stderr, flush=True)
    bwd = args.op == "backward_data"
    wgr = args.op == "backward_weight"
    inp = S.make_inputs(wl, 0, (wl.N, wl.C_out) + out_size(wl))
    if bwd:
        inp = {"dy": S.make_grad_output(wl, 0, (wl.N, wl.C_out) + out_size(wl)), "w": inp["w"]}
    elif wgr:
        inp = {"dy": S.make_grad_output(wl, 0, (wl.N, wl.C_out) + out_size(wl)), "x": inp["x"]}
    dev = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inp.items()}
    plan = T.plan_for(wl)
    if args.path != "auto":
        T.convt_plan_set_path(plan, args.path)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] path {path}: warm-up done, timing {args.steps} steps", file=sys.stderr,
          flush=True)

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_all0.elapsed_time(t_all1) / args.steps
    launches = np.array([a.elapsed_time(b) for a, b in ev])
    ms_launch = float(launches.mean())

    # Launches with the 256 MB last-level (Infinity) cache evicted first: a
    # 512 MB buffer is read before each timed launch, outside its events
    # (read, not written, so that no dirty lines are written back during the
    # launch; the warm, back-to-back figure above stays the headline).
    n_cold = min(args.steps, 20)
    evict = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    ev_cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_cold)]
    for i in range(n_cold):
        evict.sum()
        ev_cold[i][0].record(stream)
        step()
        ev_cold[i][1].record(stream)
    torch.cuda.synchronize()
    del evict
    cold = np.array([a.elapsed_time(b) for a, b in ev_cold])

    nbytes = (algorithmic_bytes_backward(wl) if bwd else algorithmic_bytes_weight(wl) if wgr
              else algorithmic_bytes(wl))
    flops = 2 * valid_macs(wl)
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_fp32 = flops / (PEAK_FP32_TFLOPS * 1e12)
    m = re.search(r"kernel=(\S+)", T.convt_plan_describe(plan))
    if bwd:
        m = re.search(r"input gradient: kernel=(\S+)", T.convt_plan_describe(plan))
    if wgr:
        m = re.search(r"weight gradient: kernel=(\S+)", T.convt_plan_describe(plan))
    kernel = m.group(1) if m else KERNEL_NAMES[path]
    if t_hbm >= t_fp32:
        ach = nbytes / (ms_launch * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        ach = flops / (ms_launch * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_FP32_TFLOPS, 4)}
    roof["traffic"] = traffic_for(wl.name, kernel)
    roof["kernel"] = kernel
    roof["launch_ms"] = round(ms_launch, 5)
    stats = lambda a: {"median": round(float(np.median(a)), 5), "min": round(float(a.min()), 5),
                       "max": round(float(a.max()), 5)}
    roof["launch_ms_stats"] = stats(launches)
    cold_ms = float(np.median(cold))
    roof["cold_cache"] = dict(stats(cold), launches=int(n_cold), frac=round(
        (t_hbm if t_hbm >= t_fp32 else t_fp32) / (cold_ms * 1e-3), 4))

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, op=args.op)

    line = {
        "metric": ("ConvTranspose input-gradient GB/s and valid-MAC TFLOP/s, % of roofline, 1x MI355X" if bwd
                   else "ConvTranspose weight-gradient GB/s and valid-MAC TFLOP/s, % of roofline, 1x MI355X" if wgr
                   else "ConvTranspose fwd GB/s and valid-MAC TFLOP/s, % of roofline, 1x MI355X"),
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded: x, add ~ N(0,1); w, bias ~ U(+-1/sqrt(fan_in)))",
        "config": {"workload": wl.name, "ndim": wl.ndim, "N": wl.N, "C_in": wl.C_in,
                   "C_out": wl.C_out, "groups": wl.groups, "in_size": list(wl.in_size),
                   "out_size": list(out_size(wl)), "K": list(wl.K), "stride": list(wl.stride),
                   "pad": list(wl.pad), "out_pad": list(wl.out_pad),
                   "dilation": list(wl.dilation), "bias": wl.bias, "fused": wl.fused,
                   "path": args.op if (bwd or wgr) else path, "op": args.op,
                   "parallelism": "single GPU"},
        "valid_mac_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "hbm_frac": round(t_hbm / (ms_per_step * 1e-3), 4),
        "fp32_frac": round(t_fp32 / (ms_per_step * 1e-3), 4),
        "algorithmic_bytes": nbytes, "valid_macs": flops // 2,
        "timed_wall_s": round(wall, 4), "source_sha": source_sha(),
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
