"""Exact-coverage, aliasing and determinism properties of the HIP library."""
import numpy as np
import pytest

import oracle
import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

from gpu_util import check_close, log, make, oracle_kwargs, reduced, run_gpu, supported_paths, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    S.TINY_1D,
    reduced(S.LONG_1D, N=2, in_size=(3001,)),
    reduced(S.GROUPED_3D, N=1, in_size=(4, 8, 8)),
    reduced(S.FUSED_3D, N=2, in_size=(6, 5, 7)),
    reduced(S.HEAVY_3D, N=1, in_size=(4, 6, 8)),
]
GUARD = 4099


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_redzones_and_inputs_intact(wl):
    """y is a slice of a larger sentinel-filled buffer: every element of y is
    overwritten, nothing before or after it is touched, the inputs are bitwise
    unchanged."""
    import torch
    inp = make(wl)
    dev = to_dev(inp)
    plan = T.plan_for(wl)
    n = int(np.prod(plan.y_shape()))
    for path in supported_paths(wl):
        buf = torch.full((n + 2 * GUARD + 1,), float("nan"), device="cuda")
        y = buf[GUARD + 1:GUARD + 1 + n].view(plan.y_shape())  # odd float offset: unaligned
        run_gpu(wl, dev, path, y=y)
        assert not torch.isnan(y).any().item(), path
        assert torch.isnan(buf[:GUARD + 1]).all().item(), path
        assert torch.isnan(buf[GUARD + 1 + n:]).all().item(), path
        for k in ("x", "w", "bias", "add"):
            if inp[k] is not None:
                assert np.array_equal(dev[k].cpu().numpy(), inp[k]), (path, k)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_deterministic(wl):
    """Atomic-free: two runs are bitwise equal."""
    dev = to_dev(make(wl))
    for path in supported_paths(wl):
        a = run_gpu(wl, dev, path).cpu().numpy()
        b = run_gpu(wl, dev, path).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), path


@pytest.mark.parametrize("wl", [w for w in CASES if w.fused] + [reduced(S.TINY_1D, fused=True)],
                         ids=lambda w: w.name)
def test_fused_in_place(wl):
    """add_input == y (in place) gives the same result as separate buffers."""
    inp = make(wl)
    ref = oracle.get().forward(**oracle_kwargs(wl, inp))
    for path in supported_paths(wl):
        dev = to_dev(inp)
        plan = T.plan_for(wl)
        T.convt_plan_set_path(plan, path)
        y = T.convt_forward_add_hswish(plan, dev["x"], dev["w"], dev["bias"], dev["add"],
                                       y=dev["add"])
        import torch
        torch.cuda.synchronize()
        check_close(y.cpu().numpy(), ref, f"{wl.name} in-place {path}")


def test_unaligned_input_pointers():
    """x, w, bias and add at odd float offsets inside larger buffers."""
    import torch
    wl = reduced(S.FUSED_3D, N=1, in_size=(3, 4, 5))
    inp = make(wl)
    ref = oracle.get().forward(**oracle_kwargs(wl, inp))

    def offset_copy(a):
        buf = torch.zeros(a.size + 3, device="cuda")
        v = buf[1:1 + a.size].view(a.shape)
        v.copy_(torch.from_numpy(a))
        return v

    dev = {k: (None if v is None else offset_copy(v)) for k, v in inp.items()}
    for path in supported_paths(wl):
        y = run_gpu(wl, dev, path)
        check_close(y.cpu().numpy(), ref, f"unaligned inputs {path}")


def test_streams():
    """The call runs on the stream it is given."""
    import torch
    wl = reduced(S.LONG_1D, N=1, in_size=(2000,))
    inp = make(wl)
    dev = to_dev(inp)
    plan = T.plan_for(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = T.convt_forward(plan, dev["x"], dev["w"], dev["bias"])
    s.synchronize()
    ref = oracle.get().forward(**oracle_kwargs(wl, inp))
    check_close(y.cpu().numpy(), ref, "side stream")
    log("  side stream ok")
