"""Channels-last layout (convt_plan_set_layout: x (N, L_in..., C_in), y and
add_input (N, L_out..., C_out)) through the C ABI against the oracle in the
same layout, element by element: reduced shapes of every workload and the
random and degenerate shapes on every path that takes them, every epilogue
mode, full sizes of the long 1D, fused 3D and channel-heavy 3D layers, and the properties that
every output element is written and the inputs are left as they were.
Inputs are the seeded channels-first draws with the channel axis moved last.
Tolerance as the forward: |got - ref| <= 1e-4 + 1e-4 |ref|."""
import numpy as np
import pytest

import oracle
import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

from gpu_util import check_close, log, make, reduced
from test_parity_gpu import DEGENERATE, REDUCED, _random_cases

pytestmark = pytest.mark.gpu

ACT_CODE = {"none": 0, "hardswish": 1, "x_hardswish": 2}


def _last(a):
    return None if a is None else np.ascontiguousarray(np.moveaxis(a, 1, -1))


def _paths(plan):
    out = []
    for name in ("generic", "stream1d", "igemm3d"):
        if T.lib().convt_plan_set_path(plan.handle, T.PATHS[name]) == T.CONVT_OK:
            out.append(name)
    T.convt_plan_set_path(plan, "auto")
    return out


def _check(wl, modes=None, paths=None, seed=0):
    import torch
    orc = oracle.get()
    inp = make(wl, seed)
    x, add = _last(inp["x"]), _last(inp["add"])
    if add is None:
        out = orc.output_size(wl.ndim, wl.in_size, wl.K, wl.stride, wl.pad, wl.out_pad, wl.dilation)
        add = _last((3 * S.normal((wl.N, wl.C_out) + out, seed, wl.wid, S.TENSOR_ADD)).astype(np.float32))
    if modes is None:
        modes = [(True, "x_hardswish")] if wl.fused else [(False, "none")]
    plan = T.plan_for(wl, "channels_last")
    kw = dict(ndim=wl.ndim, N=wl.N, C_in=wl.C_in, C_out=wl.C_out, groups=wl.groups, in_size=wl.in_size,
              K=wl.K, stride=wl.stride, pad=wl.pad, out_pad=wl.out_pad, dilation=wl.dilation, x=x, w=inp["w"],
              bias=inp["bias"], layout=1)
    dx, dw, da = (torch.from_numpy(v).cuda() for v in (x, inp["w"], add))
    db = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).cuda()
    for path in (paths or _paths(plan)):
        T.convt_plan_set_path(plan, path)
        for has_add, act in modes:
            ref = orc.forward(add=add if has_add else None, act=ACT_CODE[act], **kw)
            y = torch.full(plan.y_shape(), float("nan"), device="cuda")
            log(f"  gpu channels-last: {wl.name} N={wl.N} in={wl.in_size} path={path} add={has_add} act={act}")
            T.convt_forward_epilogue(plan, dx, dw, db, da if has_add else None, act, y=y)
            torch.cuda.synchronize()
            err = check_close(y.cpu().numpy(), ref, f"{wl.name} channels-last path={path} add={has_add} act={act}")
            log(f"  max abs err {err:.3e}")
    assert np.array_equal(dx.cpu().numpy(), x) and np.array_equal(da.cpu().numpy(), add)


@pytest.mark.parametrize("wl", REDUCED, ids=lambda w: f"{w.name}-N{w.N}-in{'x'.join(map(str, w.in_size))}")
def test_channels_last_reduced_all_paths(wl):
    _check(wl)


@pytest.mark.parametrize("wl", _random_cases(24) + DEGENERATE, ids=lambda w: w.name)
def test_channels_last_random_and_degenerate(wl):
    _check(wl)


# Shapes for the channels-last fast kernels: the long 1D layer's variants
# (several tiles per wave, ragged tails, groups, output padding, empty
# phases) and the fused 3D layer.
NLC_1D = [
    reduced(S.LONG_1D, N=2, in_size=(4099,)),
    S.Workload("nlc_chain", 1, 2, 32, 64, 1, (65553,), (3,), (2,), (1,), (0,), (2,), True, False, wid=5001),
    S.Workload("nlc_g2", 1, 3, 64, 128, 2, (517,), (3,), (2,), (2,), (1,), (2,), True, True, wid=5002),
    S.Workload("nlc_k4s2d1", 1, 1, 32, 32, 1, (777,), (4,), (2,), (1,), (0,), (1,), False, True, wid=5003),
    S.Workload("nlc_k3s3d2", 1, 2, 16, 16, 1, (300,), (3,), (3,), (2,), (1,), (2,), True, False, wid=5004),
    S.Workload("nlc_k5s4d2", 1, 1, 16, 32, 1, (257,), (5,), (4,), (3,), (2,), (2,), True, True, wid=5005),
    S.Workload("nlc_short", 1, 3, 32, 64, 1, (5,), (3,), (2,), (1,), (0,), (2,), True, False, wid=5006),
    S.Workload("nlc_L1", 1, 2, 32, 64, 1, (1,), (3,), (2,), (1,), (0,), (2,), True, False, wid=5007),
    S.Workload("nlc_32", 1, 2, 32, 32, 1, (4099,), (3,), (2,), (1,), (0,), (2,), True, True, wid=5008),
    S.Workload("nlc_chain_32", 1, 1, 32, 32, 1, (65553,), (3,), (2,), (2,), (1,), (2,), False, False, wid=5009),
]


@pytest.mark.parametrize("wl", NLC_1D, ids=lambda w: f"{w.name}-N{w.N}-in{w.in_size[0]}")
def test_channels_last_1d_fast_kernel(wl):
    plan = T.plan_for(wl, "channels_last")
    assert "kernel=k_stream1d_nlc" in T.convt_plan_describe(plan)
    _check(wl, paths=["stream1d"])


# Shapes for the channels-last implicit-GEMM kernel (weights in registers):
# fused or not, one or two W-blocks per row, a ragged last W-block, other
# paddings, 16 -> 32 channels with kernel 4, 2D.
NDHWC_3D = [
    reduced(S.FUSED_3D, N=2),
    S.Workload("ndhwc_k3s2_fused_w8", 3, 2, 32, 64, 1, (5, 7, 8), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1),
               (1, 1, 1), True, True, wid=5201),
    S.Workload("ndhwc_k3s2_w24", 3, 1, 32, 64, 1, (3, 4, 24), (3, 3, 3), (2, 2, 2), (1, 0, 1), (0, 1, 1),
               (1, 1, 1), True, False, wid=5202),
    S.Workload("ndhwc_k4s2_c16", 3, 2, 16, 32, 1, (4, 5, 20), (4, 4, 4), (2, 2, 2), (1, 1, 1), (0, 0, 0),
               (1, 1, 1), True, True, wid=5203),
    S.Workload("ndhwc_k3s2_p2", 3, 1, 32, 64, 1, (4, 4, 16), (3, 3, 3), (2, 2, 2), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), False, False, wid=5204),
    S.Workload("ndhwc_k3s2_w20", 3, 1, 32, 64, 1, (2, 3, 20), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1),
               (1, 1, 1), True, True, wid=5205),
    S.Workload("nhwc_2d_k3s2", 2, 2, 32, 64, 1, (16, 16), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), True, True,
               wid=5206),
]


@pytest.mark.parametrize("wl", NDHWC_3D, ids=lambda w: f"{w.name}-N{w.N}-in{'x'.join(map(str, w.in_size))}")
def test_channels_last_3d_fast_kernel(wl):
    plan = T.plan_for(wl, "channels_last")
    assert "kernel=k_igemm3d" in T.convt_plan_describe(plan)
    _check(wl, paths=["igemm3d"])


# Shapes for the channels-last streamed-weight kernel: the channel-heavy
# layer reduced, kernel 3 with 64 input channels, 32-channel blocks, groups,
# rows in W segments with ragged ends, 2D.
NDHWC_WIDE = [
    reduced(S.HEAVY_3D, N=1, in_size=(3, 4, 32)),
    S.Workload("ndhwc_w_k3_c64_fused", 3, 2, 64, 64, 1, (3, 5, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=5301),
    S.Workload("ndhwc_w_co32_w12", 3, 1, 32, 32, 1, (2, 5, 12), (4, 4, 4), (2, 2, 2), (1, 1, 2),
               (0, 1, 0), (1, 1, 1), True, False, wid=5302),
    S.Workload("ndhwc_w_g2_co128", 3, 1, 64, 256, 2, (2, 3, 20), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), True, False, wid=5303),
    S.Workload("ndhwc_w_seg_w44", 3, 1, 64, 64, 1, (2, 3, 44), (4, 4, 4), (2, 2, 2), (1, 1, 2),
               (0, 0, 0), (1, 1, 1), False, True, wid=5304),
    S.Workload("nhwc_w_seg_w100_co96", 2, 1, 48, 96, 1, (5, 100), (3, 3), (2, 2), (1, 2), (0, 1),
               (1, 1), True, True, wid=5305),
    S.Workload("ndhwc_w_s1w_fused", 3, 1, 64, 64, 1, (2, 3, 24), (3, 3, 3), (2, 1, 1), (1, 1, 1),
               (1, 0, 0), (1, 1, 1), True, True, wid=5306),
    S.Workload("ndhwc_w_co48", 3, 1, 64, 48, 1, (2, 3, 44), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=5307),
]


@pytest.mark.parametrize("wl", NDHWC_WIDE, ids=lambda w: f"{w.name}-N{w.N}-in{'x'.join(map(str, w.in_size))}")
def test_channels_last_wide_kernel(wl):
    plan = T.plan_for(wl, "channels_last")
    assert "kernel=k_igemm3d_wide" in T.convt_plan_describe(plan)
    _check(wl, paths=["igemm3d"])


MODES = [(add, act) for add in (False, True) for act in ("none", "hardswish", "x_hardswish")]


@pytest.mark.parametrize("wl", [S.Workload("nlc_epi", 1, 2, 32, 64, 1, (20001,), (3,), (2,), (1,), (0,), (2,),
                                           True, False, wid=5101),
                                reduced(S.FUSED_3D, N=1, in_size=(5, 7, 8)),
                                reduced(S.GROUPED_3D, N=1, in_size=(4, 8, 16)),
                                reduced(S.HEAVY_3D, N=1, in_size=(2, 3, 12))],
                         ids=lambda w: w.name)
def test_channels_last_epilogue_modes(wl):
    _check(wl, modes=MODES)


@pytest.mark.parametrize("wl", [S.LONG_1D, S.FUSED_3D, S.HEAVY_3D], ids=lambda w: w.name)
def test_channels_last_full_size_every_element(wl):
    """Full size, the planner's channels-last path (the one the bench times),
    every element against the oracle's full forward."""
    _check(wl, paths=[T.convt_plan_get_path(T.plan_for(wl, "channels_last"))])


def test_channels_last_rejects_gradients():
    import torch
    wl = reduced(S.LONG_1D, N=1, in_size=(64,))
    plan = T.plan_for(wl, "channels_last")
    dy = torch.zeros(plan.y_shape(), device="cuda")
    w = torch.zeros(plan.w_shape(), device="cuda")
    with pytest.raises(T.ConvtError) as e:
        T.convt_backward_data(plan, dy, w, dx=torch.empty(plan.x_shape(), device="cuda"))
    assert e.value.status == T.CONVT_ERR_UNSUPPORTED
