"""Weight and bias gradients (convt_backward_weight) through the C ABI against
the oracle (oracle_convt_backward_weight), element by element, on seeded
inputs: reduced shapes of every workload, the seeded random and degenerate
shapes of the forward tests, and full spatial sizes at a reduced batch.

Tolerance, derived from the arithmetic: each dw element is a sum of products
accumulated in fp32, first along a chain of MFMA steps per range of
positions, then across the ranges by atomic adds.  The general kernel runs at
most 256 four-product steps per range of 1024 positions; the LDS-staged and
window kernels up to 512 per range of 2048.  With u = 2^-24 and S = the sum
of |x * dy| over the same terms (the oracle's gradient of |x| and |dy|), the
rounding error is within (chain length) * u * S; the test allows
  |got - ref| <= 1e-4 + (max(256 + N*ceil(P/1024), 512 + N*ceil(P/2048)) + 12) * 2^-24 * S
for P input positions, whichever of those kernels runs.  The shift-pair
kernel (groups of 8 and 8 channels, stride 2 along W) accumulates in one wave
at most R * ceil((W_in + 1)/4) steps for R = D_in * H_in input rows, and at
most N * R partial sums meet by atomic adds; its row-sharing variant (H
stride 1) pads each wave's rows by up to 12, so where either runs the chain is
R * (ceil((W_in + 1)/4) + N) + 12 * (ceil((W_in + 1)/4) + 1) if that is longer.  At full spatial size that
bound is loose (S grows with the positions summed), so the same shapes also
run on small-integer inputs, where every fp32 partial sum is exact and the
result must equal the oracle's bit for bit: one dropped or doubled term
fails.
db sums N * L_out values in chunks of 16384 positions: a thread adds up to 4
values into each of 16 partial sums, which a 4-level tree, a wave tree of 6
levels and a 2-level tree across the 4 waves combine, and the N * chunks
partial sums meet by atomic adds, so
chain = ceil(min(L_out, 16384) / 4096) + 4 + 8 + N * ceil(L_out / 16384)
with S = sum |dy|."""
import numpy as np
import pytest

import oracle
import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

from gpu_util import log, reduced
from test_parity_gpu import DEGENERATE, REDUCED, _random_cases

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _kw(wl):
    return dict(ndim=wl.ndim, N=wl.N, C_in=wl.C_in, C_out=wl.C_out, groups=wl.groups, in_size=wl.in_size,
                K=wl.K, stride=wl.stride, pad=wl.pad, out_pad=wl.out_pad, dilation=wl.dilation)


def _check(wl, seed=0):
    import torch
    orc = oracle.get()
    out = orc.output_size(wl.ndim, wl.in_size, wl.K, wl.stride, wl.pad, wl.out_pad, wl.dilation)
    x = S.make_inputs(wl, seed, (wl.N, wl.C_out) + out)["x"]
    dy = S.make_grad_output(wl, seed, (wl.N, wl.C_out) + out)
    ref_w, ref_b = orc.backward_weight(x=x, dy=dy, **_kw(wl))
    abs_w, abs_b = orc.backward_weight(x=np.abs(x), dy=np.abs(dy), **_kw(wl))
    plan = T.plan_for(wl)
    log(f"  gpu backward_weight: {wl.name} N={wl.N} in={wl.in_size}")
    dx_, ddy = torch.from_numpy(x).cuda(), torch.from_numpy(dy).cuda()
    dw = torch.full(plan.w_shape(), float("nan"), dtype=torch.float32, device="cuda")
    db = torch.full((wl.C_out,), float("nan"), dtype=torch.float32, device="cuda")
    T.convt_backward_weight(plan, dx_, ddy, dw=dw, db=db)
    torch.cuda.synchronize()
    in_sp = int(np.prod(wl.in_size))
    out_sp = int(np.prod(out))
    chain_w = max(256 + wl.N * -(-in_sp // 1024), 512 + wl.N * -(-in_sp // 2048)) + 12
    if "weight gradient: kernel=k_backward_weight_shift" in T.convt_plan_describe(plan):
        rows = in_sp // wl.in_size[-1]
        spr = -(-(wl.in_size[-1] + 1) // 4)
        chain_w = max(chain_w, rows * (spr + wl.N) + 12 * (spr + 1))
    if "weight gradient: kernel=k_backward_weight_stage" in T.convt_plan_describe(plan):
        # one accumulator per workgroup over the sample's blocks of 128
        # positions (32 K-steps each), then one atomic add per sample
        lead = in_sp // (wl.in_size[-1] * wl.in_size[-2])
        nhb = -(-wl.in_size[-2] // (128 // wl.in_size[-1]))
        chain_w = max(chain_w, lead * nhb * 32 + wl.N + 12)
    chain_b = -(-min(out_sp, 16384) // 4096) + 4 + 8 + wl.N * -(-out_sp // 16384)
    for what, got, ref, s_abs, chain in (("dw", dw, ref_w, abs_w, chain_w), ("db", db, ref_b, abs_b, chain_b)):
        g = got.cpu().numpy().astype(np.float64)
        assert g.shape == ref.shape and np.all(np.isfinite(g)), (what, g.shape, ref.shape)
        err = np.abs(g - ref)
        bound = 1e-4 + chain * U * s_abs
        bad = err > bound
        assert not bad.any(), (f"{wl.name} {what}: {int(bad.sum())} of {bad.size} outside; worst "
                               f"{float((err - bound).max())}")
        log(f"  {what} max abs err {err.max():.3e} (bound min {bound.min():.3e})")
    # the inputs are left as they were
    assert np.array_equal(dx_.cpu().numpy(), x) and np.array_equal(ddy.cpu().numpy(), dy)
    # without db the call leaves any bias tensor alone and computes the same dw
    dw2, none = T.convt_backward_weight(plan, dx_, ddy, with_bias=False)
    torch.cuda.synchronize()
    assert none is None
    assert np.all(np.abs(dw2.cpu().numpy() - ref_w) <= 1e-4 + chain_w * U * abs_w)


@pytest.mark.parametrize("wl", REDUCED, ids=lambda w: f"{w.name}-N{w.N}-in{'x'.join(map(str, w.in_size))}")
def test_wgrad_reduced(wl):
    _check(wl)


@pytest.mark.parametrize("wl", _random_cases(24) + DEGENERATE, ids=lambda w: w.name)
def test_wgrad_random_and_degenerate(wl):
    _check(wl)


@pytest.mark.parametrize("wl", [reduced(S.LONG_1D, N=2), reduced(S.GROUPED_3D, N=1), reduced(S.FUSED_3D, N=2),
                                reduced(S.HEAVY_3D, N=1, in_size=(8, 16, 16))],
                         ids=lambda w: f"{w.name}-N{w.N}")
def test_wgrad_full_spatial(wl):
    _check(wl)


# One-axis shapes for the window-staged weight-gradient kernel: 6 taps in two
# chunks of up to 4 (d = 1 < s: the full window); stride 3 with d = 3 and
# stride 4 with d = 8 and two groups (d a multiple of s: the window keeps
# every s-th column).  Ragged last tiles and ranges throughout.
ROW_WINDOW = [
    S.Workload("wgrad_row_k6_chunks", 1, 3, 32, 64, 1, (1000,), (6,), (2,), (2,), (1,), (1,), True, False, 51),
    S.Workload("wgrad_row_s3d3", 1, 2, 32, 64, 1, (777,), (5,), (3,), (4,), (2,), (3,), True, False, 52),
    S.Workload("wgrad_row_s4d8_g2", 1, 2, 64, 128, 2, (301,), (3,), (4,), (3,), (0,), (8,), True, False, 53),
]


@pytest.mark.parametrize("wl", ROW_WINDOW, ids=lambda w: w.name)
def test_wgrad_row_window(wl):
    assert "weight gradient: kernel=k_backward_weight_row" in T.convt_plan_describe(T.plan_for(wl))
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
def test_wgrad_leading_unit_axis(wl):
    assert "_row" not in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)


# Shapes for the shift-pair kernel (groups of 8 input and 8 output channels,
# stride 2 and dilation 1 along W): 1D and 2D, three groups, K_w = 9 (a tile
# with taps past K), K_w = 1, 40 tiles in three chunks, dilations and strides
# on D and H, a padding that crops taps, odd W.
SHIFT = [
    S.Workload("ws_1d_crop", 1, 2, 8, 8, 1, (101,), (5,), (2,), (6,), (1,), (1,), True, False, 71),
    S.Workload("ws_2d", 2, 2, 8, 8, 1, (5, 21), (3, 7), (1, 2), (1, 3), (0, 1), (1, 1), True, False, 72),
    S.Workload("ws_g3_k9", 3, 1, 24, 24, 3, (3, 4, 10), (2, 3, 9), (2, 2, 2), (0, 1, 4), (1, 1, 1), (2, 1, 1),
               True, False, 73),
    S.Workload("ws_k1", 3, 2, 8, 8, 1, (2, 3, 7), (1, 1, 1), (1, 1, 2), (0, 0, 0), (0, 0, 1), (1, 1, 1), False,
               False, 74),
    S.Workload("ws_40_tiles", 3, 1, 16, 16, 2, (3, 5, 8), (4, 5, 6), (2, 1, 2), (1, 2, 2), (1, 0, 1), (1, 2, 1),
               True, False, 75),
]


# Shapes for the row-sharing variant (H stride 1, dilation 1): H taps 1, 4
# (an odd number of dy row slots: 10 rows per unrolled trip) and 7, W taps 8
# (two T blocks) and 3 (one), H lengths that leave a short last row range,
# several samples and groups, a cropping pad.
SHIFT_ROWS = [
    S.Workload("wsr_kh7_kw8", 3, 2, 16, 16, 2, (2, 23, 12), (2, 7, 8), (2, 1, 2), (1, 3, 3), (1, 0, 1),
               (1, 1, 1), True, False, 76),
    S.Workload("wsr_kh4_kw3", 3, 3, 8, 8, 1, (3, 31, 9), (3, 4, 3), (1, 1, 2), (1, 1, 1), (0, 0, 1), (2, 1, 1),
               False, False, 77),
    S.Workload("wsr_kh1_crop", 2, 2, 8, 8, 1, (13, 40), (1, 5), (1, 2), (0, 6), (0, 1), (1, 1), True, False, 78),
]


@pytest.mark.parametrize("wl", SHIFT_ROWS, ids=lambda w: w.name)
def test_wgrad_shift_rows(wl):
    assert "weight gradient: kernel=k_backward_weight_shift_rows" in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)
    _check_exact(wl)


# Shapes for the LDS-staged weight kernel (groups of 32k input and 4k output
# channels, W_in of 16, 32 or 64, at most 32 taps): the fused layer's
# geometry with H 20 (a partial last block of 4 rows); W 32 with two groups,
# H dilation 2 and 16 taps (four waves without a tap group); 2D with W 64 and
# W stride 3; one D tap with D stride 3, W dilation 3 and two channel
# chunks; 32 taps (every wave has a group).
WT_STAGE = [
    S.Workload("wst_w16_h20", 3, 2, 32, 8, 1, (2, 20, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 0, 1), (1, 1, 1),
               True, False, 101),
    S.Workload("wst_w32_g2_dh2", 3, 1, 64, 8, 2, (2, 5, 32), (2, 2, 4), (1, 2, 2), (0, 1, 2), (0, 1, 1),
               (1, 2, 1), True, False, 102),
    S.Workload("wst_2d_w64_s3", 2, 2, 32, 4, 1, (7, 64), (3, 2), (1, 3), (1, 0), (0, 2), (1, 1), False, False, 103),
    S.Workload("wst_kd1_dw3", 3, 1, 64, 12, 1, (4, 9, 16), (1, 3, 2), (3, 1, 3), (0, 1, 2), (2, 0, 1), (1, 1, 3),
               True, False, 104),
    S.Workload("wst_taps32", 3, 1, 32, 8, 1, (3, 8, 16), (2, 4, 4), (1, 1, 1), (1, 2, 1), (0, 0, 0), (1, 1, 1),
               True, False, 105),
    # two tap groups per wave: 48 taps (waves 4-7 have no second group) with
    # W 32; the channel-heavy layer's geometry (64 taps, W 32, stride 2) with a
    # partial last block of 2 rows, two channel chunks and 8 output channels
    S.Workload("wst_taps48", 3, 1, 32, 8, 1, (3, 6, 32), (3, 4, 4), (2, 1, 2), (1, 1, 1), (1, 0, 1), (1, 1, 1),
               True, False, 106),
    S.Workload("wst_heavy_geo", 3, 1, 64, 8, 1, (3, 6, 32), (4, 4, 4), (2, 2, 2), (1, 1, 1), (0, 0, 0), (1, 1, 1),
               True, False, 107),
]


@pytest.mark.parametrize("wl", WT_STAGE, ids=lambda w: w.name)
def test_wgrad_stage(wl):
    assert "weight gradient: kernel=k_backward_weight_stage" in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)
    _check_exact(wl)


@pytest.mark.parametrize("wl", SHIFT, ids=lambda w: w.name)
def test_wgrad_shift_pairs(wl):
    assert "weight gradient: kernel=k_backward_weight_shift" in T.convt_plan_describe(T.plan_for(wl))
    _check(wl)
    _check_exact(wl)


def _check_exact(wl, seed=0):
    """x and dy small integers in [-3, 3]: every product and partial sum is an
    integer below 2^24 in magnitude (at most 9 * N * P for dw and 3 * N * L_out
    for db), so fp32 represents each exactly and the GPU must match the fp64
    oracle exactly."""
    import torch
    orc = oracle.get()
    out = orc.output_size(wl.ndim, wl.in_size, wl.K, wl.stride, wl.pad, wl.out_pad, wl.dilation)
    in_sp, out_sp = int(np.prod(wl.in_size)), int(np.prod(out))
    assert 9 * wl.N * in_sp < 2 ** 24 and 3 * wl.N * out_sp < 2 ** 24
    x = S.small_integers(wl.x_shape(), 3, seed, wl.wid, S.TENSOR_X)
    dy = S.small_integers((wl.N, wl.C_out) + tuple(out), 3, seed, wl.wid, S.TENSOR_DY)
    ref_w, ref_b = orc.backward_weight(x=x, dy=dy, **_kw(wl))
    plan = T.plan_for(wl)
    log(f"  gpu backward_weight (integer inputs): {wl.name} N={wl.N} in={wl.in_size}")
    dw = torch.full(plan.w_shape(), float("nan"), dtype=torch.float32, device="cuda")
    db = torch.full((wl.C_out,), float("nan"), dtype=torch.float32, device="cuda")
    T.convt_backward_weight(plan, torch.from_numpy(x).cuda(), torch.from_numpy(dy).cuda(), dw=dw, db=db)
    torch.cuda.synchronize()
    for what, got, ref in (("dw", dw, ref_w), ("db", db, ref_b)):
        g = got.cpu().numpy().astype(np.float64)
        bad = g != ref
        assert not bad.any(), (f"{wl.name} {what}: {int(bad.sum())} of {bad.size} differ; worst "
                               f"{float(np.abs(g - ref).max())}")


@pytest.mark.parametrize("wl", [reduced(S.LONG_1D, N=2), reduced(S.GROUPED_3D, N=1), reduced(S.FUSED_3D, N=2),
                                reduced(S.HEAVY_3D, N=1, in_size=(8, 16, 16))],
                         ids=lambda w: f"{w.name}-N{w.N}")
def test_wgrad_full_spatial_exact(wl):
    _check_exact(wl)
