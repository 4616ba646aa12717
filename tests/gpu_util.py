"""Helpers for the GPU tests: run the HIP library through its C ABI on seeded
inputs and compare with the oracle.  Tolerance (fp32 path vs fp64 oracle):
|got - ref| <= ATOL + RTOL*|ref| elementwise, ATOL = RTOL = 1e-4."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle
import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

ATOL = 1e-4
RTOL = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_kwargs(wl: S.Workload, inp):
    return dict(ndim=wl.ndim, N=wl.N, C_in=wl.C_in, C_out=wl.C_out, groups=wl.groups,
                in_size=wl.in_size, K=wl.K, stride=wl.stride, pad=wl.pad, out_pad=wl.out_pad,
                dilation=wl.dilation, x=inp["x"], w=inp["w"], bias=inp["bias"], add=inp["add"])


def make(wl: S.Workload, seed: int = 0):
    """Seeded inputs; add_input shaped by the oracle's own output size."""
    out = oracle.get().output_size(wl.ndim, wl.in_size, wl.K, wl.stride, wl.pad, wl.out_pad,
                                   wl.dilation)
    return S.make_inputs(wl, seed, (wl.N, wl.C_out) + out)


def to_dev(inp):
    import torch
    return {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inp.items()}


def run_gpu(wl: S.Workload, dev, path: str = "auto", y=None):
    """One forward (fused if the workload is) through the C ABI; returns y."""
    plan = T.plan_for(wl)
    if path != "auto":
        T.convt_plan_set_path(plan, path)
    log(f"  gpu run: {wl.name} path={T.convt_plan_get_path(plan)}")
    if wl.fused:
        y = T.convt_forward_add_hswish(plan, dev["x"], dev["w"], dev["bias"], dev["add"], y=y)
    else:
        y = T.convt_forward(plan, dev["x"], dev["w"], dev["bias"], y=y)
    import torch
    torch.cuda.synchronize()
    return y


def check_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst flat "
                             f"index {i}: got {got.ravel()[i]!r} ref {ref.ravel()[i]!r}")
    return float(err.max()) if err.size else 0.0


def supported_paths(wl: S.Workload):
    plan = T.plan_for(wl)
    out = []
    for name in ("generic", "stream1d", "igemm3d"):
        if T.lib().convt_plan_set_path(plan.handle, T.PATHS[name]) == T.CONVT_OK:
            out.append(name)
    return out


def sample_indices(wl: S.Workload, out_size, n_random: int, seed: int = 1):
    """Flat output indices: random ones plus every combination of the first
    and last positions of each axis for a few (n, co)."""
    rng = np.random.default_rng(seed)
    total = wl.N * wl.C_out * int(np.prod(out_size))
    idx = [rng.integers(0, total, size=n_random)]
    edges = [sorted(set([0, 1, 2, 3, L - 4, L - 3, L - 2, L - 1]) & set(range(L))) for L in out_size]
    for n in sorted({0, wl.N - 1}):
        for co in sorted({0, wl.C_out // 2, wl.C_out - 1}):
            base = (n * wl.C_out + co)
            grids = np.meshgrid(*edges, indexing="ij")
            flat = np.zeros_like(grids[0], dtype=np.int64)
            for a, g in enumerate(grids):
                flat = flat * out_size[a] + g
            idx.append(base * int(np.prod(out_size)) + flat.ravel())
    return np.unique(np.concatenate(idx).astype(np.int64))


def reduced(wl: S.Workload, **kw) -> S.Workload:
    return dataclasses.replace(wl, **kw)
