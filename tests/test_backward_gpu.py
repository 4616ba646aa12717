"""Input gradient (convt_backward_data) through the C ABI against the oracle's
adjoint loop (oracle_convt_backward_data), element by element, on seeded
inputs: reduced shapes of every workload, the seeded random and degenerate
shapes of the forward tests, full spatial sizes at a reduced batch, and the
properties that every dx element is written and the inputs are untouched.
Tolerance as the forward: |got - ref| <= 1e-4 + 1e-4 |ref|."""
import numpy as np
import pytest

import oracle
import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

from gpu_util import check_close, log, reduced
from test_parity_gpu import DEGENERATE, REDUCED, _random_cases

pytestmark = pytest.mark.gpu


def _inputs(wl, seed):
    """dy ~ N(0, 1) in the forward output's shape and w as the workload's,
    from the seeded generators both sides use."""
    out = oracle.get().output_size(wl.ndim, wl.in_size, wl.K, wl.stride, wl.pad, wl.out_pad, wl.dilation)
    inp = S.make_inputs(wl, seed, (wl.N, wl.C_out) + out)
    return S.make_grad_output(wl, seed, (wl.N, wl.C_out) + out), inp["w"]


def _check(wl, seed=0):
    import torch
    dy, w = _inputs(wl, seed)
    ref = oracle.get().backward_data(ndim=wl.ndim, N=wl.N, C_in=wl.C_in, C_out=wl.C_out, groups=wl.groups,
                                     in_size=wl.in_size, K=wl.K, stride=wl.stride, pad=wl.pad,
                                     out_pad=wl.out_pad, dilation=wl.dilation, dy=dy, w=w)
    plan = T.plan_for(wl)
    log(f"  gpu backward_data: {wl.name} N={wl.N} in={wl.in_size}")
    ddy, dw = torch.from_numpy(dy).cuda(), torch.from_numpy(w).cuda()
    dx = torch.full(plan.x_shape(), float("nan"), dtype=torch.float32, device="cuda")
    T.convt_backward_data(plan, ddy, dw, dx=dx)
    torch.cuda.synchronize()
    err = check_close(dx.cpu().numpy(), ref, f"backward_data {wl.name}")
    log(f"  max abs err {err:.3e}")
    # the inputs are left as they were
    assert np.array_equal(ddy.cpu().numpy(), dy) and np.array_equal(dw.cpu().numpy(), w)


@pytest.mark.parametrize("wl", REDUCED, ids=lambda w: f"{w.name}-N{w.N}-in{'x'.join(map(str, w.in_size))}")
def test_backward_reduced(wl):
    _check(wl)


@pytest.mark.parametrize("wl", _random_cases(24) + DEGENERATE, ids=lambda w: w.name)
def test_backward_random_and_degenerate(wl):
    _check(wl)


@pytest.mark.parametrize("wl", [reduced(S.LONG_1D, N=2), reduced(S.GROUPED_3D, N=1), reduced(S.FUSED_3D, N=2),
                                reduced(S.HEAVY_3D, N=1, in_size=(8, 32, 32))],
                         ids=lambda w: f"{w.name}-N{w.N}")
def test_backward_full_spatial(wl):
    _check(wl)


# One-axis shapes for the window-staged matrix kernel.  Grids large enough
# that a workgroup walks several position tiles: 3 tiles per workgroup with a
# last workgroup of 2 and a ragged last tile (d a multiple of s: the window
# keeps every s-th column); 4 with two groups and unit stride; the cap of 8
# (d = 1 < s: the full window).  Then strides 3 and 4 with d a multiple of s,
# which the compressed window brings within its column limit.
ROW_TILES = [
    S.Workload("bwd_row_tiles3_ragged", 1, 300, 16, 4, 1, (5669,), (3,), (2,), (1,), (1,), (2,), False, False, 41),
    S.Workload("bwd_row_tiles4_g2", 1, 140, 32, 8, 2, (7683,), (4,), (1,), (2,), (0,), (3,), False, False, 42),
    S.Workload("bwd_row_tiles8", 1, 700, 16, 4, 1, (5889,), (3,), (2,), (0,), (0,), (1,), False, False, 43),
    S.Workload("bwd_row_s3d3", 1, 2, 16, 8, 1, (700,), (3,), (3,), (2,), (1,), (3,), False, False, 44),
    S.Workload("bwd_row_s4d8_g2", 1, 3, 32, 16, 2, (301,), (5,), (4,), (7,), (2,), (8,), False, False, 45),
]


@pytest.mark.parametrize("wl", ROW_TILES, ids=lambda w: w.name)
def test_backward_row_multitile(wl):
    assert "input gradient: kernel=k_backward_data_mfma_row" in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)


# 2D shapes whose leading axis has one input position and one tap, with a
# padding that drops that tap (p = 1, out_pad 2: one output, no contribution,
# so the gradients of x and w are zero) or leaves it at output 0 of three
# (p = 0, out_pad 2).  They must not take the one-axis window kernels.
LEADING_UNIT_AXIS = [
    S.Workload("lead_unit_p1_op2", 2, 2, 32, 64, 1, (1, 1000), (1, 3), (3, 2), (1, 1), (2, 0), (1, 2), True, False, 61),
    S.Workload("lead_unit_p0_op2", 2, 2, 32, 64, 1, (1, 1000), (1, 3), (3, 2), (0, 1), (2, 0), (1, 2), True, False, 62),
]


@pytest.mark.parametrize("wl", LEADING_UNIT_AXIS, ids=lambda w: w.name)
def test_backward_leading_unit_axis(wl):
    assert "_row" not in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)


# Shapes for the W-pair kernel (groups of 8 input and 8 output channels,
# stride 2 and dilation 1 along W, stride 1 and dilation 1 along H): W
# tiles of 32 positions with a partial last one, H not a multiple of the
# wave's 4 rows, H taps 1, 3 and 7, W taps 1, 4 and 9, three groups, a D
# stride of 3 with dilation 2, 2D, and a weight volume near the LDS copy's
# limit (3 x 7 x 9 = 189).
BWD_WPAIR = [
    S.Workload("bwp_w33_h6", 3, 2, 8, 8, 1, (2, 6, 33), (2, 3, 4), (1, 1, 2), (0, 1, 1), (0, 0, 1), (1, 1, 1),
               False, False, 81),
    S.Workload("bwp_g3_kh7_kw9", 3, 1, 24, 24, 3, (3, 9, 40), (3, 7, 9), (2, 1, 2), (1, 3, 4), (1, 0, 1),
               (1, 1, 1), False, False, 82),
    S.Workload("bwp_kh1_kw1_d3", 3, 2, 8, 8, 1, (4, 5, 17), (2, 1, 1), (3, 1, 2), (1, 0, 0), (2, 0, 1), (2, 1, 1),
               False, False, 83),
    S.Workload("bwp_2d", 2, 3, 16, 16, 2, (7, 70), (3, 5), (1, 2), (1, 2), (0, 1), (1, 1), False, False, 84),
]


@pytest.mark.parametrize("wl", BWD_WPAIR, ids=lambda w: w.name)
def test_backward_wpair(wl):
    assert "input gradient: kernel=k_backward_data_wpair" in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)


# Shapes for the LDS-staged matrix kernel (groups of 32k input and 4k output
# channels, W_in of 16, 32 or 64, at most 64 taps): a second row block that
# is partial (H 20 with 16 rows per workgroup) and 27 taps; W 32 with two
# groups, H dilation 2 and an even tap count (16: the last tap's operand
# reads run one tap past the end); 2D with W 64, W stride 3 and one channel
# quad; one D tap with D stride 3, W dilation 3, three quads and two channel
# chunks.
BWD_STAGE = [
    S.Workload("bst_w16_h20", 3, 2, 32, 8, 1, (3, 20, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 0, 1), (1, 1, 1),
               False, False, 85),
    S.Workload("bst_w32_g2_dh2", 3, 1, 64, 16, 2, (2, 9, 32), (2, 2, 4), (1, 2, 2), (0, 1, 2), (0, 1, 1),
               (1, 2, 1), False, False, 86),
    S.Workload("bst_2d_w64_s3", 2, 2, 32, 4, 1, (7, 64), (3, 2), (1, 3), (1, 0), (0, 2), (1, 1), False, False, 87),
    S.Workload("bst_kd1_dw3", 3, 1, 64, 12, 1, (4, 5, 16), (1, 3, 2), (3, 1, 3), (0, 1, 2), (2, 0, 1), (1, 1, 3),
               False, False, 88),
    # more than 32 taps: the weights staged per (quad, D tap).  The channel-heavy
    # layer's geometry (W 32, 4 x 4 x 4 taps, stride 2) with a partial second
    # row block and two channel chunks; 48 taps with 16 per D tap on W 16.
    S.Workload("bst_heavy_geo", 3, 1, 64, 8, 1, (3, 10, 32), (4, 4, 4), (2, 2, 2), (1, 1, 1), (0, 0, 0), (1, 1, 1),
               False, False, 89),
    S.Workload("bst_taps48", 3, 1, 32, 8, 1, (3, 9, 16), (3, 4, 4), (2, 1, 2), (1, 2, 1), (1, 0, 1), (1, 1, 1),
               False, False, 120),
]


@pytest.mark.parametrize("wl", BWD_STAGE, ids=lambda w: w.name)
def test_backward_stage(wl):
    assert "input gradient: kernel=k_backward_data_stage" in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)
