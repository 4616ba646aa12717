"""The selectable epilogue (convt_forward_epilogue) through the C ABI against
the oracle, element by element: every mode (residual add or not, times the
identity, hardswish or t * hardswish(t)) on every path that accepts each
shape, with shapes that reach every kernel: the 1D streaming kernel (including
its chained common path), the implicit-GEMM kernels (weights in registers and
streamed), and the generic kernels (row pairs, rows, phase classes, and the
one-thread-per-position kernel).  Tolerance as the forward:
|got - ref| <= 1e-4 + 1e-4 |ref|."""
import numpy as np
import pytest

import oracle
import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

from gpu_util import check_close, log, make, reduced, supported_paths

pytestmark = pytest.mark.gpu

MODES = [(add, act) for add in (False, True) for act in ("none", "hardswish", "x_hardswish")]
ACT_CODE = {"none": 0, "hardswish": 1, "x_hardswish": 2}

CASES = [
    S.TINY_1D,
    reduced(S.LONG_1D, N=2, in_size=(4099,)),
    S.Workload("epi_s1d_chain", 1, 2, 32, 64, 1, (65553,), (3,), (2,), (1,), (0,), (2,), True, False, wid=4001),
    reduced(S.GROUPED_3D, N=1, in_size=(4, 8, 16)),
    reduced(S.FUSED_3D, N=1, in_size=(5, 7, 8)),
    reduced(S.HEAVY_3D, N=1, in_size=(3, 4, 32)),
    S.Workload("epi_rows", 3, 2, 24, 8, 2, (2, 11, 6), (3, 4, 2), (1, 1, 2), (1, 1, 0), (0, 0, 1), (1, 1, 1),
               True, False, wid=4002),
    # more than 32 phase classes: the one-thread-per-position kernel
    S.Workload("epi_many_classes", 3, 1, 4, 6, 1, (3, 4, 5), (4, 3, 3), (4, 3, 3), (1, 1, 1), (0, 1, 2),
               (1, 1, 1), True, False, wid=4003),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: f"{w.name}-N{w.N}-in{'x'.join(map(str, w.in_size))}")
def test_epilogue_modes_all_paths(wl):
    import torch
    orc = oracle.get()
    inp = make(wl)
    out = orc.output_size(wl.ndim, wl.in_size, wl.K, wl.stride, wl.pad, wl.out_pad, wl.dilation)
    # add_input scaled so that t spans both bends of hardswish (-3 and +3)
    add = (3 * S.normal((wl.N, wl.C_out) + out, 0, wl.wid, S.TENSOR_ADD)).astype(np.float32)
    kw = dict(ndim=wl.ndim, N=wl.N, C_in=wl.C_in, C_out=wl.C_out, groups=wl.groups, in_size=wl.in_size,
              K=wl.K, stride=wl.stride, pad=wl.pad, out_pad=wl.out_pad, dilation=wl.dilation,
              x=inp["x"], w=inp["w"], bias=inp["bias"])
    dx, dw = torch.from_numpy(inp["x"]).cuda(), torch.from_numpy(inp["w"]).cuda()
    db = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).cuda()
    da = torch.from_numpy(add).cuda()
    plan = T.plan_for(wl)
    for path in supported_paths(wl):
        T.convt_plan_set_path(plan, path)
        for has_add, act in MODES:
            ref = orc.forward(add=add if has_add else None, act=ACT_CODE[act], **kw)
            y = torch.full(plan.y_shape(), float("nan"), device="cuda")
            T.convt_forward_epilogue(plan, dx, dw, db, da if has_add else None, act, y=y)
            torch.cuda.synchronize()
            err = check_close(y.cpu().numpy(), ref, f"{wl.name} path={path} add={has_add} act={act}")
            log(f"  {wl.name} path={path} add={has_add} act={act}: max abs err {err:.3e}")


def test_epilogue_matches_fixed_entry_points():
    """convt_forward is the epilogue call with no add and no activation,
    convt_forward_add_hswish the one with add and t * hardswish(t): bitwise."""
    import torch
    for wl in (reduced(S.LONG_1D, N=2, in_size=(4099,)), reduced(S.FUSED_3D, N=1, in_size=(5, 7, 8))):
        inp = make(wl)
        plan = T.plan_for(wl)
        out = plan.out_size
        add = torch.from_numpy(S.normal((wl.N, wl.C_out) + out, 0, wl.wid, S.TENSOR_ADD)).cuda()
        dx, dw = torch.from_numpy(inp["x"]).cuda(), torch.from_numpy(inp["w"]).cuda()
        db = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).cuda()
        a = T.convt_forward(plan, dx, dw, db)
        b = T.convt_forward_epilogue(plan, dx, dw, db, None, "none")
        c = T.convt_forward_add_hswish(plan, dx, dw, db, add)
        d = T.convt_forward_epilogue(plan, dx, dw, db, add, "x_hardswish")
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(c, d), wl.name
