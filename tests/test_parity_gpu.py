"""Parity of the HIP library (through its C ABI) with the CPU oracle.

* Reduced shapes of every workload (several tiles, ragged tails): every
  element against the oracle's full forward, on every path that supports the
  shape.
* A seeded sweep of small random shapes (1D/2D/3D, groups, stride, padding,
  output padding, dilation, bias, fused) and degenerate shapes.
* Full-size workloads in the configuration the bench times: sampled outputs
  against the oracle's one-by-one evaluation, plus exact properties.
"""
import numpy as np
import pytest

import oracle
import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

from gpu_util import (check_close, log, make, oracle_kwargs, reduced, run_gpu, sample_indices,
                      supported_paths, to_dev)

pytestmark = pytest.mark.gpu

REDUCED = [
    S.TINY_1D,
    reduced(S.LONG_1D, N=2, in_size=(4099,)),
    reduced(S.LONG_1D, N=1, in_size=(1,)),
    reduced(S.GROUPED_3D, N=2),
    reduced(S.FUSED_3D, N=2),
    reduced(S.FUSED_3D, N=1, in_size=(5, 7, 9)),
    reduced(S.HEAVY_3D, N=1, in_size=(6, 5, 9)),
    reduced(S.HEAVY_3D, N=2, in_size=(4, 4, 16)),
    # 1D shapes for each streaming-kernel variant: groups, fused, several
    # non-empty phases, empty phases, output padding, ragged lengths
    S.Workload("s1d_g2_k3s2d2", 1, 2, 64, 128, 2, (517,), (3,), (2,), (1,), (0,), (2,), True, True,
               wid=3001),
    S.Workload("s1d_k3s2d1", 1, 2, 32, 64, 1, (1000,), (3,), (2,), (1,), (1,), (1,), True, False,
               wid=3002),
    S.Workload("s1d_k4s2d1", 1, 1, 32, 32, 1, (777,), (4,), (2,), (1,), (0,), (1,), False, True,
               wid=3003),
    S.Workload("s1d_k3s3d2", 1, 2, 16, 16, 1, (300,), (3,), (3,), (2,), (1,), (2,), True, False,
               wid=3004),
    S.Workload("s1d_k5s4d2", 1, 1, 16, 32, 1, (257,), (5,), (4,), (3,), (2,), (2,), True, True,
               wid=3005),
    S.Workload("s1d_short", 1, 3, 32, 64, 1, (5,), (3,), (2,), (1,), (0,), (2,), True, False,
               wid=3006),
    # the 64- and 32-channel variants (channels first only for 64)
    S.Workload("s1d_64_k3s2d2", 1, 2, 64, 64, 1, (517,), (3,), (2,), (1,), (0,), (2,), True, True,
               wid=3011),
    S.Workload("s1d_g2_64_k3s2d1", 1, 1, 128, 128, 2, (300,), (3,), (2,), (1,), (1,), (1,), True, False,
               wid=3012),
    S.Workload("s1d_32_k3s2d2", 1, 2, 32, 32, 1, (1000,), (3,), (2,), (2,), (1,), (2,), False, False,
               wid=3013),
    # 3D shapes for each implicit-GEMM variant: fused or not, two W-blocks per
    # row, ragged last W-block, other paddings and output paddings
    S.Workload("ig_k3s2_fused_w8", 3, 2, 32, 64, 1, (5, 7, 8), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3101),
    S.Workload("ig_k3s2_w24", 3, 1, 32, 64, 1, (3, 4, 24), (3, 3, 3), (2, 2, 2), (1, 0, 1),
               (0, 1, 1), (1, 1, 1), True, False, wid=3102),
    S.Workload("ig_k4s2_c16", 3, 2, 16, 32, 1, (4, 5, 12), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), True, True, wid=3103),
    S.Workload("ig_k3s2_p2", 3, 1, 32, 64, 1, (4, 4, 16), (3, 3, 3), (2, 2, 2), (2, 2, 2),
               (1, 1, 1), (1, 1, 1), False, False, wid=3104),
    S.Workload("ig_k3s2_w20", 3, 1, 32, 64, 1, (2, 3, 20), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3105),
    # multi-row steps (classes of one or two D x H taps take 4 or 2 rows along
    # H per step): every light class multi-row; mixed with single-row classes
    # whose H runs do not split into whole steps; two taps along D (K_H = 2)
    S.Workload("ig_multirow_fused", 3, 2, 32, 64, 1, (3, 8, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3106),
    S.Workload("ig_multirow_mixed", 3, 3, 32, 64, 1, (4, 5, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 0, 1), (1, 1, 1), True, False, wid=3107),
    S.Workload("ig_multirow_kh2", 3, 2, 32, 64, 1, (3, 8, 16), (3, 2, 3), (2, 2, 2), (1, 0, 1),
               (1, 0, 1), (1, 1, 1), False, True, wid=3108),
    # channel-heavy shapes (weights streamed through LDS): two W-blocks, a
    # ragged last W-block, 64 input channels, fused
    reduced(S.HEAVY_3D, N=1, in_size=(3, 4, 32)),
    S.Workload("igw_c128_p2", 3, 1, 128, 64, 1, (3, 3, 32), (4, 4, 4), (2, 2, 2), (2, 1, 2),
               (1, 0, 0), (1, 1, 1), True, False, wid=3201),
    S.Workload("igw_c64_fused", 3, 2, 64, 64, 1, (2, 5, 32), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), True, True, wid=3202),
    S.Workload("igw_c128_w16_nobias", 3, 1, 128, 64, 1, (5, 2, 16), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 1, 0), (1, 1, 1), False, False, wid=3203),
    # kernel 3 along W (12-byte weight loads): the fused layer's geometry with
    # 64 input channels, 128 input channels on rows of 64 outputs, a ragged
    # last W-block; kernel 4 with 32 input channels and with 64 on one W-block
    S.Workload("igw_k3_c64_fused", 3, 2, 64, 64, 1, (3, 5, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3204),
    S.Workload("igw_k3_c128_w32", 3, 1, 128, 64, 1, (2, 4, 32), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, False, wid=3205),
    S.Workload("igw_k3_c64_w24", 3, 2, 64, 64, 1, (3, 3, 24), (3, 3, 3), (2, 2, 2), (1, 0, 1),
               (0, 1, 0), (1, 1, 1), False, True, wid=3206),
    S.Workload("igw_k4_c32_fused", 3, 2, 32, 64, 1, (3, 4, 32), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), True, True, wid=3207),
    S.Workload("igw_k4_c32_w12", 3, 1, 32, 64, 1, (2, 5, 12), (4, 4, 4), (2, 2, 2), (1, 1, 2),
               (0, 1, 0), (1, 1, 1), True, False, wid=3208),
    S.Workload("igw_k4_c64_w16", 3, 1, 64, 64, 1, (2, 3, 16), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), False, False, wid=3209),
    # output channels in blocks of 32 (64 -> 32, 48 -> 96: three blocks, three
    # input-channel chunks) and of 64 (64 -> 128: two blocks); 16 input
    # channels; stride 1 on D and H (3 and 4 taps per class, 12 tap slots)
    S.Workload("igw_co32_k3_fused", 3, 2, 64, 32, 1, (3, 4, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3210),
    S.Workload("igw_co128_k4", 3, 1, 64, 128, 1, (2, 3, 32), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), True, False, wid=3211),
    S.Workload("igw_co96_c48", 3, 1, 48, 96, 1, (2, 3, 20), (3, 3, 3), (2, 2, 2), (1, 1, 0),
               (0, 1, 1), (1, 1, 1), True, False, wid=3212),
    S.Workload("igw_c16_k3_fused", 3, 2, 16, 64, 1, (3, 3, 8), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3213),
    S.Workload("igw_s1_taps12", 3, 1, 64, 64, 1, (4, 5, 16), (3, 4, 3), (1, 1, 2), (1, 1, 1),
               (0, 0, 1), (1, 1, 1), False, True, wid=3214),
    # groups: 32 channels per group (32-channel blocks), 32 -> 128 per group
    # (two 64-channel blocks per group)
    S.Workload("igw_g2_co32_fused", 3, 2, 64, 64, 2, (3, 4, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3216),
    S.Workload("igw_g2_co128_k4", 3, 1, 64, 256, 2, (2, 3, 20), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), True, False, wid=3217),
    # stride 1 along W with kernel 3 (taps at shifts 0..2): two W-blocks, a
    # ragged one-block row with 3 D taps per class
    S.Workload("igw_s1w_k3_fused", 3, 2, 64, 64, 1, (3, 4, 20), (3, 3, 3), (2, 2, 1), (1, 1, 1),
               (1, 1, 0), (1, 1, 1), True, True, wid=3218),
    S.Workload("igw_s1w_p0_co64", 3, 1, 32, 64, 1, (2, 3, 12), (3, 3, 3), (1, 2, 1), (0, 0, 0),
               (0, 0, 0), (1, 1, 1), True, False, wid=3219),
    # output channels in blocks of 16 (64 -> 16 on the fused geometry, 64 -> 48
    # in three blocks with kernel 4, stride 1 with 2 groups of 64 -> 16)
    S.Workload("igw_co16_fused", 3, 2, 64, 16, 1, (3, 4, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 1, 1), (1, 1, 1), True, True, wid=3220),
    S.Workload("igw_co48_k4_w24", 3, 1, 64, 48, 1, (2, 3, 24), (4, 4, 4), (2, 2, 2), (1, 1, 1),
               (0, 0, 0), (1, 1, 1), True, False, wid=3221),
    S.Workload("igw_co16_g2_s1w", 3, 1, 128, 32, 2, (2, 3, 36), (3, 3, 3), (2, 1, 1), (1, 1, 1),
               (1, 0, 0), (1, 1, 1), False, True, wid=3222),
    # rows longer than 32 inputs in W segments of 32 (halo staged per
    # segment): two segments with a ragged last one
    S.Workload("igw_seg_w44_k4", 3, 1, 64, 64, 1, (2, 3, 44), (4, 4, 4), (2, 2, 2), (1, 1, 2),
               (0, 0, 0), (1, 1, 1), True, False, wid=3215),
    # generic path on the matrix cores with input rows shared along H (the
    # 4x4x1 rows kernel or, for groups of 8k output and 4k input channels, the
    # 16x16x4 row-pair kernel): two H tap counts (one launch each) and a ragged
    # last row block, a partial input-channel chunk, 4-channel blocks with a
    # partial chunk, bias-only classes (H stride above K), two channel chunks,
    # 2D, and an H dilation that sends the shape to the FMA phase kernel
    S.Workload("rows_hs2_g2", 3, 2, 16, 16, 2, (3, 7, 9), (3, 3, 3), (2, 2, 2), (1, 1, 1),
               (1, 0, 1), (1, 1, 1), True, False, wid=3401),
    S.Workload("rows_cig4", 3, 1, 8, 16, 2, (4, 9, 10), (2, 5, 3), (2, 1, 2), (0, 2, 1),
               (0, 0, 1), (1, 1, 1), True, True, wid=3402),
    S.Workload("rows_cpt4_cig12", 3, 2, 24, 8, 2, (2, 11, 6), (3, 4, 2), (1, 1, 2), (1, 1, 0),
               (0, 0, 1), (1, 1, 1), False, False, wid=3403),
    S.Workload("rows_bias_only", 3, 1, 8, 8, 1, (3, 6, 5), (1, 2, 3), (1, 3, 2), (0, 0, 1),
               (0, 2, 0), (1, 1, 1), True, True, wid=3404),
    S.Workload("rows_cig16", 3, 1, 32, 16, 2, (2, 8, 12), (3, 5, 3), (1, 1, 2), (1, 2, 1),
               (0, 0, 1), (1, 1, 1), True, False, wid=3405),
    S.Workload("rows_2d", 2, 3, 16, 24, 2, (13, 17), (5, 4), (1, 2), (2, 1), (0, 1), (1, 1),
               True, True, wid=3406),
    S.Workload("rows_hdil2", 3, 1, 8, 8, 1, (3, 9, 8), (3, 3, 3), (2, 1, 2), (1, 2, 1),
               (1, 0, 1), (1, 2, 1), True, False, wid=3407),
    S.Workload("rows_cig6", 3, 2, 12, 16, 2, (3, 10, 7), (2, 3, 3), (2, 1, 2), (0, 1, 1),
               (1, 0, 1), (1, 1, 1), True, True, wid=3408),
    # 8-channel groups with stride 2 along W, the two W phases in one tile
    # (k_generic_wpair): groups of P1's layer at reduced size with a ragged H
    # run (7 rows), W kernel 4 (one phase's taps all at other shifts), an odd
    # output width, two groups with bias-only D classes, fused
    S.Workload("wpair_g1_h7", 3, 1, 8, 8, 1, (3, 7, 8), (3, 5, 7), (2, 1, 2), (1, 2, 3), (1, 0, 1),
               (1, 1, 1), True, False, wid=3411),
    S.Workload("wpair_kw4_fused", 3, 2, 8, 8, 1, (2, 7, 16), (2, 3, 4), (1, 2, 2), (0, 1, 1), (0, 1, 0),
               (1, 1, 1), True, True, wid=3412),
    S.Workload("wpair_odd_w", 3, 2, 16, 16, 2, (3, 5, 12), (3, 5, 5), (2, 1, 2), (1, 2, 2), (1, 0, 0),
               (1, 1, 1), False, False, wid=3413),
    S.Workload("wpair_sd4", 3, 1, 16, 16, 2, (2, 6, 8), (3, 5, 7), (4, 1, 2), (1, 2, 3), (0, 0, 1),
               (1, 1, 1), True, True, wid=3414),
    # 8-channel groups on 16x16x4 tiles of two output rows: two channel
    # chunks, ragged position and row blocks, fused
    S.Workload("pairs_co16_ragged", 3, 2, 8, 32, 2, (3, 13, 21), (3, 5, 3), (2, 1, 2), (1, 2, 1),
               (1, 0, 0), (1, 1, 1), True, True, wid=3409),
    S.Workload("pairs_2d_k4", 2, 2, 16, 8, 1, (15, 40), (4, 3), (1, 2), (1, 1), (0, 1), (1, 1),
               False, False, wid=3410),
    # ConvTranspose2d on the implicit-GEMM kernels (depth-1 3D problems):
    # weights in registers, fused or not, and weights streamed
    S.Workload("ig2d_k3s2_fused", 2, 2, 32, 64, 1, (16, 16), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1),
               True, True, wid=3301),
    S.Workload("ig2d_k3s2_w24", 2, 3, 32, 64, 1, (7, 24), (3, 3), (2, 2), (1, 0), (0, 1), (1, 1),
               True, False, wid=3302),
    S.Workload("igw2d_c128_k4", 2, 2, 128, 64, 1, (9, 32), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1),
               True, False, wid=3303),
    S.Workload("igw2d_c64_k3", 2, 2, 64, 64, 1, (10, 20), (3, 3), (2, 2), (1, 1), (1, 0), (1, 1),
               True, True, wid=3304),
    S.Workload("igw2d_co32_k4", 2, 2, 32, 32, 1, (12, 32), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1),
               True, False, wid=3305),
    # 2D rows in W segments: 64 inputs (two segments), 100 inputs in 32-channel
    # blocks (four, the last 6 outputs), W padding 3 (later first positions)
    S.Workload("igw2d_seg_w64_k3", 2, 2, 32, 64, 1, (6, 64), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1),
               True, True, wid=3306),
    S.Workload("igw2d_seg_w100_co32", 2, 1, 64, 32, 1, (5, 100), (3, 3), (2, 2), (1, 2), (0, 1),
               (1, 1), True, True, wid=3307),
    S.Workload("igw2d_seg_p3", 2, 2, 16, 64, 1, (4, 68), (4, 4), (2, 2), (1, 3), (1, 1), (1, 1),
               False, False, wid=3308),
    S.Workload("igw2d_g4_seg", 2, 1, 64, 128, 4, (5, 44), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1),
               True, True, wid=3309),
    S.Workload("igw2d_s1w_seg_co32", 2, 1, 32, 32, 1, (6, 52), (3, 3), (1, 1), (1, 1), (0, 0), (1, 1),
               True, False, wid=3310),
]


def _full_check(wl, path):
    inp = make(wl)
    ref = oracle.get().forward(**oracle_kwargs(wl, inp))
    y = run_gpu(wl, to_dev(inp), path)
    err = check_close(y.cpu().numpy(), ref, f"{wl.name} {wl.in_size} N={wl.N} path={path}")
    log(f"  max abs err {err:.3e}")


@pytest.mark.parametrize("wl", REDUCED, ids=lambda w: f"{w.name}-N{w.N}-in{'x'.join(map(str, w.in_size))}")
def test_reduced_workloads_all_paths(wl):
    for path in supported_paths(wl):
        _full_check(wl, path)


def _random_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        nd = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 1, 2, 4]))
        Cig = int(rng.choice([1, 3, 4, 8, 16]))
        Cog = int(rng.choice([1, 2, 5, 16, 32]))
        K = tuple(int(v) for v in rng.integers(1, 6, nd))
        s = tuple(int(v) for v in rng.integers(1, 4, nd))
        d = tuple(int(v) for v in rng.integers(1, 3, nd))
        p = tuple(int(rng.integers(0, d[a] * (K[a] - 1) + 2)) for a in range(nd))
        op = tuple(int(rng.integers(0, s[a] + 1)) for a in range(nd))
        if nd == 1:
            ins = (int(rng.integers(1, 200)),)
        elif nd == 2:
            ins = tuple(int(v) for v in rng.integers(1, 14, 2))
        else:
            ins = tuple(int(v) for v in rng.integers(1, 8, 3))
        outs = [(ins[a] - 1) * s[a] - 2 * p[a] + d[a] * (K[a] - 1) + op[a] + 1 for a in range(nd)]
        if min(outs) < 1:
            continue
        wl = S.Workload(f"rand{len(out)}", nd, int(rng.integers(1, 3)), G * Cig, G * Cog, G, ins, K,
                        s, p, op, d, bool(rng.integers(0, 2)), bool(rng.integers(0, 2)),
                        wid=1000 + len(out))
        out.append(wl)
    return out


@pytest.mark.parametrize("wl", _random_cases(24), ids=lambda w: w.name)
def test_random_shapes_all_paths(wl):
    log(f"  case {wl}")
    for path in supported_paths(wl):
        _full_check(wl, path)


DEGENERATE = [
    # L_in = 1, K = 1, s = 1 (a plain 1x1 channel mix)
    S.Workload("k1s1", 1, 2, 8, 16, 1, (1,), (1,), (1,), (0,), (0,), (1,), True, False, wid=2001),
    # stride larger than the dilated kernel: most phases empty -> bias only
    S.Workload("s_gt_k", 1, 1, 4, 16, 1, (37,), (2,), (5,), (0,), (4,), (1,), True, False, wid=2002),
    # padding cropping every tap of the first inputs
    S.Workload("p_gt_span", 1, 1, 4, 16, 1, (40,), (3,), (2,), (5,), (1,), (2,), True, True, wid=2003),
    # depthwise groups
    S.Workload("depthwise3d", 3, 2, 8, 8, 8, (3, 4, 5), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1),
               (1, 1, 1), True, False, wid=2004),
    # output padding >= stride
    S.Workload("op_ge_s", 2, 1, 4, 4, 1, (5, 6), (3, 2), (2, 1), (1, 0), (3, 2), (1, 1), False, True,
               wid=2005),
    # single input and output channel, long ragged row
    S.Workload("c1_long", 1, 3, 1, 1, 1, (1001,), (3,), (2,), (1,), (1,), (2,), True, False, wid=2006),
]


@pytest.mark.parametrize("wl", DEGENERATE, ids=lambda w: w.name)
def test_degenerate_shapes(wl):
    for path in supported_paths(wl):
        _full_check(wl, path)


# Workgroups walking chains of several items (the 1D kernel's common path,
# with each row's first outputs carried from the item before), and the output
# placed 0..3 floats past an allocation's start so that other row alignments
# occur: one non-empty phase with three paddings and an output padding, and
# both phases non-empty.
CHAINED_1D = [
    S.Workload("s1d_chain_p1", 1, 2, 32, 64, 1, (65553,), (3,), (2,), (1,), (0,), (2,), True, False,
               wid=3007),
    S.Workload("s1d_chain_p2_op1", 1, 2, 32, 64, 1, (65553,), (3,), (2,), (2,), (1,), (2,), True,
               False, wid=3008),
    S.Workload("s1d_chain_p3", 1, 1, 32, 64, 1, (65553,), (3,), (2,), (3,), (0,), (2,), False, False,
               wid=3009),
    S.Workload("s1d_chain_d1", 1, 2, 32, 64, 1, (65553,), (3,), (2,), (1,), (1,), (1,), True, False,
               wid=3010),
    S.Workload("s1d_chain_64", 1, 1, 64, 64, 1, (65553,), (3,), (2,), (1,), (0,), (2,), True, False,
               wid=3014),
    S.Workload("s1d_chain_32", 1, 2, 32, 32, 1, (65553,), (3,), (2,), (1,), (0,), (2,), True, False,
               wid=3015),
    S.Workload("s1d_chain_64_d1", 1, 1, 64, 64, 1, (65553,), (3,), (2,), (1,), (1,), (1,), True, False,
               wid=3016),
]


@pytest.mark.parametrize("shift", [0, 1, 3])
@pytest.mark.parametrize("wl", CHAINED_1D, ids=lambda w: w.name)
def test_chained_1d_offset_output(wl, shift):
    import torch
    inp = make(wl)
    dev = to_dev(inp)
    plan = T.plan_for(wl)
    assert T.convt_plan_get_path(plan) == "stream1d"
    numel = wl.N * wl.C_out * plan.out_size[0]
    base = torch.full((numel + 4,), float("nan"), device="cuda")
    y = base[shift:shift + numel].view((wl.N, wl.C_out) + plan.out_size)
    y = run_gpu(wl, dev, "auto", y=y)
    assert torch.isnan(base[:shift]).all().item() and torch.isnan(base[shift + numel:]).all().item(), \
        "written outside the output"
    ref = oracle.get().forward(**oracle_kwargs(wl, inp))
    err = check_close(y.cpu().numpy(), ref, f"{wl.name} output at +{shift} floats")
    log(f"  {wl.name} +{shift}: max abs err {err:.3e}")


FULL = [S.TINY_1D, S.LONG_1D, S.GROUPED_3D, S.FUSED_3D, S.HEAVY_3D]


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_full_size_sampled(wl):
    """Full size, planner's path (the one the bench times): coverage (a NaN
    sentinel must be overwritten everywhere), sampled values vs the oracle's
    one-by-one evaluation, inputs untouched."""
    import torch
    inp = make(wl)
    dev = to_dev(inp)
    plan = T.plan_for(wl)
    y = torch.full((wl.N, wl.C_out) + plan.out_size, float("nan"), device="cuda")
    y = run_gpu(wl, dev, "auto", y=y)
    assert not torch.isnan(y).any().item(), "some output element was not written"
    assert torch.isfinite(y).all().item()
    idx = sample_indices(wl, plan.out_size, 3000)
    got = y.view(-1)[torch.from_numpy(idx).cuda()].cpu().numpy()
    ref = oracle.get().points(idx, **oracle_kwargs(wl, inp))
    err = check_close(got, ref, f"{wl.name} sampled ({idx.size} points)")
    log(f"  {wl.name}: path={T.convt_plan_get_path(plan)} max abs err {err:.3e} over {idx.size} samples")
    for k in ("x", "w", "bias", "add"):
        if inp[k] is not None:
            assert np.array_equal(dev[k].cpu().numpy(), inp[k]), f"{k} was modified"


def test_full_size_long1d_even_outputs_exactly_zero():
    """Stride 2, padding 1, dilation 2, no bias: every even output position
    receives no tap and must be exactly 0 ("Kimi-K2.6 l1_p79" transcript, the
    odd-position analysis)."""
    import torch
    wl = S.LONG_1D
    dev = to_dev(make(wl))
    y = run_gpu(wl, dev)
    assert (y[:, :, 0::2] == 0).all().item()
    assert (y[:, :, 1::2] != 0).float().mean().item() > 0.99


@pytest.mark.parametrize("wl", [S.LONG_1D, S.GROUPED_3D, S.FUSED_3D, S.HEAVY_3D], ids=lambda w: w.name)
def test_full_size_every_element(wl):
    """Full size, planner's path, every element against the oracle's full
    forward (the channel-heavy 3D layer's 131 G multiply-adds take the
    oracle about 15 s on 8 host threads; the others a few seconds)."""
    inp = make(wl)
    y = run_gpu(wl, to_dev(inp), "auto").cpu().numpy()
    ref = oracle.get().forward(**oracle_kwargs(wl, inp))
    err = check_close(y, ref, f"{wl.name} full")
    log(f"  {wl.name}: every element, max abs err {err:.3e}")
