"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and its host-only calls (plan creation, validation, output size,
path forcing, description) behave as documented.  No compute call is made."""
import ctypes
import json
import os
import re

import pytest

import transposed_convolution_forward_amd as T
from transposed_convolution_forward_amd import synthetic as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convt.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CONVT_API\s+[\w\s\*]*?\b(convt_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    declared = header_functions()
    assert len(declared) >= 9
    L = T.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(T.EXPORTS) == declared


def _create(ndim=1, N=1, C_in=2, C_out=2, groups=1, in_size=(4,), K=(3,), s=(2,), p=(1,), op=(0,),
            d=(1,)):
    L = T.lib()
    h = ctypes.c_void_p()
    arr = lambda v: (ctypes.c_int64 * len(v))(*v)
    st = L.convt_plan_create(ctypes.byref(h), ndim, N, C_in, C_out, groups, arr(in_size), arr(K),
                             arr(s), arr(p), arr(op), arr(d))
    if st == 0:
        L.convt_plan_destroy(h)
    return st


@pytest.mark.parametrize("kw,status", [
    (dict(), T.CONVT_OK),
    (dict(ndim=0), T.CONVT_ERR_INVALID_ARG),
    (dict(ndim=4, in_size=(2,) * 4, K=(1,) * 4, s=(1,) * 4, p=(0,) * 4, op=(0,) * 4, d=(1,) * 4),
     T.CONVT_ERR_INVALID_ARG),
    (dict(N=0), T.CONVT_ERR_INVALID_ARG),
    (dict(C_in=0), T.CONVT_ERR_INVALID_ARG),
    (dict(C_in=3, groups=2), T.CONVT_ERR_INVALID_ARG),
    (dict(C_out=3, groups=2), T.CONVT_ERR_INVALID_ARG),
    (dict(groups=0), T.CONVT_ERR_INVALID_ARG),
    (dict(K=(0,)), T.CONVT_ERR_INVALID_ARG),
    (dict(s=(0,)), T.CONVT_ERR_INVALID_ARG),
    (dict(d=(0,)), T.CONVT_ERR_INVALID_ARG),
    (dict(p=(-1,)), T.CONVT_ERR_INVALID_ARG),
    (dict(op=(-1,)), T.CONVT_ERR_INVALID_ARG),
    (dict(in_size=(0,)), T.CONVT_ERR_INVALID_ARG),
    # L_out = (1-1)*1 - 2*2 + 1*(3-1) + 0 + 1 = -1
    (dict(in_size=(1,), s=(1,), p=(2,)), T.CONVT_ERR_INVALID_ARG),
    # L_out = 1 exactly is valid
    (dict(in_size=(1,), K=(1,), s=(1,), p=(0,)), T.CONVT_OK),
    (dict(op=(7,)), T.CONVT_OK),          # out_pad >= stride is accepted
    (dict(p=(9,), in_size=(16,)), T.CONVT_OK),  # p > d(K-1): crops real taps
    (dict(K=(33,)), T.CONVT_ERR_UNSUPPORTED),
    (dict(s=(33,)), T.CONVT_ERR_UNSUPPORTED),
    (dict(in_size=(1 << 31,)), T.CONVT_ERR_UNSUPPORTED),
    # a huge dilation cancelled by a huge padding: L_out = 3, but the
    # uncropped length 2*(2^31 - 1) + 1 overflows the kernels' int indices
    (dict(K=(3,), d=((1 << 31) - 1,), p=((1 << 31) - 1,), in_size=(2,), s=(1,)), T.CONVT_ERR_UNSUPPORTED),
    # the same uncropped length just within the limit is accepted
    (dict(K=(3,), d=((1 << 30) - 2,), p=((1 << 30) - 2,), in_size=(2,), s=(1,)), T.CONVT_OK),
])
def test_plan_create_validation(kw, status):
    assert _create(**kw) == status


def test_null_arguments():
    L = T.lib()
    arr = (ctypes.c_int64 * 1)(4)
    assert L.convt_plan_create(None, 1, 1, 1, 1, 1, arr, arr, arr, arr, arr, arr) == T.CONVT_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert L.convt_plan_create(ctypes.byref(h), 1, 1, 1, 1, 1, None, arr, arr, arr, arr, arr) == T.CONVT_ERR_INVALID_ARG
    L.convt_plan_destroy(None)  # no-op
    assert L.convt_plan_output_size(None, arr) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_forward(None, None, None, None, None, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_forward_add_hswish(None, None, None, None, None, None, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_forward_epilogue(None, None, None, None, None, 0, None, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_backward_data(None, None, None, None, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_backward_weight(None, None, None, None, None, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_plan_set_path(None, 0) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_plan_describe(None, None, 0) == -1


def test_forward_rejects_null_tensors_without_launch():
    p = T.Plan(1, 1, 2, 2, 1, (4,), (3,), (2,), (1,), (0,), (1,))
    L = T.lib()
    fake = ctypes.c_void_p(16)  # never dereferenced: the NULL check comes first
    assert L.convt_forward(p.handle, None, fake, None, fake, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_forward(p.handle, fake, None, None, fake, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_forward(p.handle, fake, fake, None, None, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_forward_add_hswish(p.handle, fake, fake, None, None, fake, None) == T.CONVT_ERR_INVALID_ARG
    # the selectable epilogue: NULL x, w or y, or an activation outside the enum
    assert L.convt_forward_epilogue(p.handle, None, fake, None, None, 0, fake, None) == T.CONVT_ERR_INVALID_ARG
    assert L.convt_forward_epilogue(p.handle, fake, fake, None, None, 0, None, None) == T.CONVT_ERR_INVALID_ARG
    for bad in (-1, 3, 99):
        assert L.convt_forward_epilogue(p.handle, fake, fake, None, None, bad, fake, None) == T.CONVT_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert T.convt_status_string(s)
    assert T.convt_status_string(99) == "unknown status"


def test_output_sizes_match_pages():
    data = json.load(open(os.path.join(ROOT, "tests", "golden", "closed_form_and_tap_counts.json")))
    for e in data["output_sizes"]:
        nd = len(e["in_size"])
        p = T.Plan(nd, 1, 1, 1, 1, e["in_size"], e["K"], e["stride"], e["pad"], e["out_pad"],
                   e["dilation"])
        assert list(p.out_size) == e["out_size"], e["citation"]


def test_workload_plans_and_paths():
    want = {S.TINY_1D.name: (129,), S.LONG_1D.name: (262145,), S.GROUPED_3D.name: (32, 32, 64),
            S.FUSED_3D.name: (32, 32, 32), S.HEAVY_3D.name: (64, 64, 64)}
    for wl in S.WORKLOADS:
        p = T.plan_for(wl)
        assert p.out_size == want[wl.name]
        assert T.convt_plan_get_path(p) in ("generic", "stream1d", "igemm3d")
        T.convt_plan_set_path(p, "generic")
        assert T.convt_plan_get_path(p) == "generic"
        T.convt_plan_set_path(p, "auto")
        text = T.convt_plan_describe(p)
        assert "path=" in text and "r0:" in text
        kern = {"generic": "k_generic", "stream1d": "k_stream1d"}.get(T.convt_plan_get_path(p))
        assert ("kernel=" + kern) in text if kern else ("kernel=k_igemm3d" in text)
    # the channel-heavy layer streams its weights through LDS
    assert "kernel=k_igemm3d_wide" in T.convt_plan_describe(T.plan_for(S.HEAVY_3D))
    assert "kernel=k_igemm3d\n" in T.convt_plan_describe(T.plan_for(S.FUSED_3D))
    # few stride-phase classes: the phase-class gather, on the matrix cores with
    # input rows shared along H where the shape has H extent; the tiny 1D layer
    # (two classes, no H) takes the FMA variant
    # 8-channel groups with stride 2 along W: the two W phases share a tile
    assert "kernel=k_generic_wpair" in T.convt_plan_describe(T.plan_for(S.GROUPED_3D))
    # the same groups with stride 1 along W: row pairs along H
    w1 = T.Plan(3, 1, 32, 32, 4, (4, 6, 16), (3, 5, 3), (2, 1, 1), (1, 2, 1), (1, 0, 0), (1, 1, 1))
    assert "kernel=k_generic_pairs" in T.convt_plan_describe(w1)
    assert "kernel=k_generic_phase" in T.convt_plan_describe(T.plan_for(S.TINY_1D))
    # more classes than the table holds (4*3*3 = 36): the per-position gather
    big = T.Plan(3, 1, 2, 2, 1, (4, 4, 4), (4, 3, 3), (4, 3, 3), (0, 0, 0), (0, 0, 0), (1, 1, 1))
    assert "kernel=k_generic\n" in T.convt_plan_describe(big)
    # 2D plans with the implicit-GEMM channel counts take those kernels
    p2 = T.Plan(2, 2, 32, 64, 1, (16, 16), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1))
    assert T.convt_plan_get_path(p2) == "igemm3d"
    assert "kernel=k_igemm3d\n" in T.convt_plan_describe(p2)
    p2w = T.Plan(2, 2, 128, 64, 1, (9, 32), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1))
    assert "kernel=k_igemm3d_wide" in T.convt_plan_describe(p2w)
    # kernel 3 or 4 with stride 2 along W (rows of any length that is a
    # multiple of 4, in segments) streams the weights for any input channel
    # count that is a multiple of 16 and output channels in blocks of 64 or 32:
    # 64 -> 64 on the fused layer's geometry,
    # 128 -> 64 with kernel 3, 32 -> 64 with kernel 4 (no weights-in-VGPR
    # variant), 64 -> 32, 48 -> 96, 64 -> 128, strides 1 on D and H
    for cin, cout, k, s_dh in ((64, 64, 3, 2), (128, 64, 3, 2), (32, 64, 4, 2), (64, 64, 4, 2),
                               (64, 32, 3, 2), (48, 96, 4, 2), (64, 128, 3, 2), (16, 64, 3, 2),
                               (64, 64, 3, 1), (32, 32, 4, 1)):
        for w_in in (16, 32, 64, 132):
            pw = T.Plan(3, 2, cin, cout, 1, (8, 8, w_in), (k,) * 3, (s_dh, s_dh, 2), (1, 1, 1),
                        (1, 1, 1) if k == 3 and s_dh == 2 else (0, 0, 0), (1, 1, 1))
            assert "kernel=k_igemm3d_wide" in T.convt_plan_describe(pw), (cin, cout, k, s_dh, w_in)
    # kernel 3 with stride 1 along W (one W phase, taps at shifts 0..2)
    for cin, cout in ((64, 64), (32, 32), (128, 64)):
        for w_in in (12, 32, 100):
            ps = T.Plan(3, 2, cin, cout, 1, (8, 8, w_in), (3, 3, 3), (2, 2, 1), (1, 1, 1), (1, 1, 0), (1, 1, 1))
            assert "kernel=k_igemm3d_wide" in T.convt_plan_describe(ps), (cin, cout, w_in)
    # 16-channel output blocks with 64 or more input channels; below that the
    # generic kernels
    for cin, cout, wide in ((64, 16, True), (64, 48, True), (128, 80, True), (32, 48, False), (16, 16, False)):
        pc = T.Plan(3, 2, cin, cout, 1, (8, 8, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), (1, 1, 1))
        assert ("kernel=k_igemm3d_wide" in T.convt_plan_describe(pc)) == wide, (cin, cout)
    # groups whose channel counts fit (16k inputs, 32k outputs per group) too
    for cin, cout, g in ((64, 64, 2), (64, 256, 2), (64, 128, 4)):
        pg = T.Plan(3, 2, cin, cout, g, (8, 8, 16), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), (1, 1, 1))
        assert "kernel=k_igemm3d_wide" in T.convt_plan_describe(pg), (cin, cout, g)
    # rows whose length is not a multiple of 4, output channels not in blocks
    # of 16, input channels not in chunks of 16, more than 4 taps per class on
    # D do not
    for a in (((8, 8, 50), 64, 64, (3, 3, 3), (2, 2, 2)), ((8, 8, 16), 64, 40, (3, 3, 3), (2, 2, 2)),
              ((8, 8, 16), 24, 64, (3, 3, 3), (2, 2, 2)), ((8, 8, 16), 64, 64, (5, 3, 3), (1, 2, 2))):
        ins, cin, cout, k, st = a
        text = T.convt_plan_describe(T.Plan(3, 2, cin, cout, 1, ins, k, st, (1, 1, 1), (0, 1, 1), (1, 1, 1)))
        assert "kernel=k_igemm3d" not in text, a
    # P1's grouped layer (8 channels per group) keeps its W-pair kernel
    assert "kernel=k_igemm3d" not in T.convt_plan_describe(T.plan_for(S.GROUPED_3D))

def _gradient_kernels(plan):
    text = T.convt_plan_describe(plan)
    return tuple(line.split("=")[1] for line in text.splitlines() if "gradient: kernel=" in line)


def test_gradient_kernel_routing():
    """The describe text names the kernels the gradient calls run; the
    choices follow the kernels' documented conditions."""
    want = {S.TINY_1D.name: ("k_backward_data", "k_backward_weight"),
            S.LONG_1D.name: ("k_backward_data_mfma_row", "k_backward_weight_row"),
            S.GROUPED_3D.name: ("k_backward_data_wpair", "k_backward_weight_shift_rows"),
            S.FUSED_3D.name: ("k_backward_data_stage", "k_backward_weight_stage"),
            S.HEAVY_3D.name: ("k_backward_data_stage", "k_backward_weight_stage")}
    for wl in S.WORKLOADS:
        assert _gradient_kernels(T.plan_for(wl)) == want[wl.name], wl.name
    # one axis, s = 3 and d = 2: the input gradient's full window (765 + 5
    # columns) exceeds its 640-column limit, the weight gradient's (194) fits
    p = T.Plan(1, 2, 32, 64, 1, (1000,), (3,), (3,), (1,), (0,), (2,))
    assert _gradient_kernels(p) == ("k_backward_data_mfma", "k_backward_weight_row")
    # d a multiple of s: only every s-th column is kept, and both windows fit
    p = T.Plan(1, 2, 32, 64, 1, (1000,), (3,), (3,), (1,), (0,), (3,))
    assert _gradient_kernels(p) == ("k_backward_data_mfma_row", "k_backward_weight_row")
    # s = 4, d = 1, K = 5: the weight gradient's window (256 columns) does not
    # fit 64 KB of LDS beside the x tile
    p = T.Plan(1, 2, 32, 64, 1, (1000,), (5,), (4,), (1,), (0,), (1,))
    assert _gradient_kernels(p) == ("k_backward_data_mfma", "k_backward_weight_lds")
    # 4 output channels per group: the window kernel's 4-channel chunks still
    # apply; the weight gradient's channel blocks do not
    p = T.Plan(1, 2, 16, 4, 1, (1000,), (3,), (2,), (1,), (0,), (2,))
    assert _gradient_kernels(p) == ("k_backward_data_mfma_row", "k_backward_weight")
    # a 2D plan whose leading axis has one input and one tap but a padding
    # that drops that tap (L_out = 1) or more than one output: the window
    # kernels index only the last axis, so neither may take it
    for lead_p, lead_op in ((1, 2), (0, 2)):
        p = T.Plan(2, 2, 32, 64, 1, (1, 1000), (1, 3), (3, 2), (lead_p, 1), (lead_op, 0), (1, 2))
        assert _gradient_kernels(p) == ("k_backward_data_mfma", "k_backward_weight_lds"), (lead_p, lead_op)
    # the shift-pair weight kernel needs groups of 8 and 8 channels, stride 2 and
    # dilation 1 along W: stride 1, dilation 2 or 16 output channels per group
    # take the general kernel
    for s_w, d_w, cout in ((2, 1, 32), (1, 1, 32), (2, 2, 32), (2, 1, 64)):
        p = T.Plan(3, 1, 32, cout, 4, (4, 6, 16), (3, 5, 7), (2, 1, s_w), (1, 2, 3), (1, 0, 1), (1, 1, d_w))
        want = "k_backward_weight_shift_rows" if (s_w, d_w, cout) == (2, 1, 32) else "k_backward_weight"
        assert _gradient_kernels(p)[1] == want, (s_w, d_w, cout)
        # the input gradient's W-pair kernel has the same conditions (and H
        # stride and dilation 1, which these plans have)
        want = "k_backward_data_wpair" if (s_w, d_w, cout) == (2, 1, 32) else "k_backward_data"
        assert _gradient_kernels(p)[0] == want, (s_w, d_w, cout)
    # the LDS-staged input gradient: 32 input channels per group and at most
    # 64 taps (16 per D tap above 32); 16 channels per group, 72 taps or W 48
    # take the matrix kernel
    for cin, k_w, w_in in ((32, 3, 16), (16, 3, 16), (32, 8, 16), (32, 3, 48)):
        p = T.Plan(3, 2, cin, 64, 1, (16, 16, w_in), (3, 3, k_w), (2, 2, 2), (1, 1, 1), (1, 1, 1), (1, 1, 1))
        want = "k_backward_data_stage" if (cin, k_w, w_in) == (32, 3, 16) else "k_backward_data_mfma"
        assert _gradient_kernels(p)[0] == want, (cin, k_w, w_in)
        # the staged weight kernel has the same conditions but up to 64 taps
        # (the 72 here take the LDS kernel); otherwise 64 output channels take
        # the LDS kernel when the input channels fill it
        want = ("k_backward_weight_stage" if (cin, k_w, w_in) == (32, 3, 16)
                else "k_backward_weight" if cin == 16 else "k_backward_weight_lds")
        assert _gradient_kernels(p)[1] == want, (cin, k_w, w_in)
    # past the staged kernels' window buffers: H stride 3 on W_in 16 needs 4 x 48
    # x 33 = 6336 window floats for the input gradient (over 4608); W_in 64 needs
    # 3 x 4 x 5 x 129 = 7740 for the weight gradient's D taps (over 7168)
    p = T.Plan(3, 2, 32, 64, 1, (8, 16, 16), (3, 3, 3), (2, 3, 2), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert _gradient_kernels(p)[0] == "k_backward_data_mfma"
    p = T.Plan(3, 2, 32, 64, 1, (8, 4, 64), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert _gradient_kernels(p)[1] == "k_backward_weight_lds"
    # H stride 2: not the W-pair input-gradient kernel, and the weight gradient
    # without row sharing
    p = T.Plan(3, 1, 32, 32, 4, (4, 6, 16), (3, 5, 7), (2, 2, 2), (1, 2, 3), (1, 1, 1), (1, 1, 1))
    assert _gradient_kernels(p) == ("k_backward_data", "k_backward_weight_shift")
    # 9 W taps (three T blocks): the weight gradient without row sharing
    p = T.Plan(3, 1, 32, 32, 4, (4, 6, 16), (3, 5, 9), (2, 1, 2), (1, 2, 4), (1, 0, 1), (1, 1, 1))
    assert _gradient_kernels(p)[1] == "k_backward_weight_shift"


def test_phase_table_description():
    # stride 2, padding 1, dilation 2, kernel 3: residue 0 takes every tap, residue 1 none
    p = T.Plan(1, 1, 1, 1, 1, (8,), (3,), (2,), (1,), (0,), (2,))
    text = T.convt_plan_describe(p)
    assert "r0:{k0/c0,k1/c1,k2/c2} r1:{}" in text


def test_set_path_rejects_unsupported():
    p = T.Plan(1, 1, 2, 3, 1, (8,), (3,), (2,), (1,), (0,), (1,))
    assert T.lib().convt_plan_set_path(p.handle, 7) == T.CONVT_ERR_INVALID_ARG
    assert T.convt_plan_get_path(p) == "generic"
    assert T.lib().convt_plan_set_path(p.handle, T.PATHS["igemm3d"]) == T.CONVT_ERR_UNSUPPORTED


def test_layout_selection():
    """channels last re-plans: the long 1D layer takes its channels-last
    streaming kernel, other shapes the channels-last generic kernel; the
    gradient kernels are not offered; bad values are rejected."""
    p = T.plan_for(S.LONG_1D)
    assert T.convt_plan_get_layout(p) == "channels_first"
    T.convt_plan_set_layout(p, "channels_last")
    assert T.convt_plan_get_layout(p) == "channels_last"
    text = T.convt_plan_describe(p)
    assert "layout=channels_last" in text and "kernel=k_stream1d_nlc" in text and "gradient" not in text
    assert p.x_shape() == (16, 131072, 32) and p.y_shape() == (16, 262145, 64)
    q = T.plan_for(S.GROUPED_3D, "channels_last")
    assert "kernel=k_generic_nxc" in T.convt_plan_describe(q)
    # the channel-heavy layer streams its weights in either layout
    assert "kernel=k_igemm3d_wide" in T.convt_plan_describe(T.plan_for(S.HEAVY_3D, "channels_last"))
    assert T.lib().convt_plan_set_layout(q.handle, 2) == T.CONVT_ERR_INVALID_ARG
    assert T.lib().convt_plan_set_layout(None, 1) == T.CONVT_ERR_INVALID_ARG
    assert T.lib().convt_plan_get_layout(None) == -1
    T.convt_plan_set_layout(p, "channels_first")
    assert "kernel=k_stream1d\n" in T.convt_plan_describe(p)
    # the 64-channel streaming variants are compiled for channels first only;
    # the 32 -> 32 one for both layouts
    w64 = T.Plan(1, 2, 64, 64, 1, (517,), (3,), (2,), (1,), (0,), (2,))
    assert "kernel=k_stream1d\n" in T.convt_plan_describe(w64)
    T.convt_plan_set_layout(w64, "channels_last")
    assert "kernel=k_generic_nxc" in T.convt_plan_describe(w64)
    w32 = T.Plan(1, 2, 32, 32, 1, (517,), (3,), (2,), (1,), (0,), (2,))
    assert "kernel=k_stream1d\n" in T.convt_plan_describe(w32)
    T.convt_plan_set_layout(w32, "channels_last")
    assert "kernel=k_stream1d_nlc" in T.convt_plan_describe(w32)


def test_convt_log_names_kernel_and_fallback():
    """CONVT_LOG=1: one stderr line per plan with the chosen kernel, and the
    generic fallback called out (a subprocess, so the variable is read at
    plan creation)."""
    import subprocess
    import sys
    code = ("import transposed_convolution_forward_amd as T; from transposed_convolution_forward_amd import "
            "synthetic as S; T.plan_for(S.LONG_1D); T.plan_for(S.GROUPED_3D); "
            "T.Plan(1, 1, 64, 64, 1, (100,), (4,), (2,), (1,), (0,), (1,))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       env={**os.environ, "CONVT_LOG": "1"})
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("convt: plan:")]
    assert len(lines) == 3, r.stderr
    assert "kernel=k_stream1d" in lines[0] and "fallback" not in lines[0]
    assert "kernel=k_generic_wpair" in lines[1] and "generic fallback" in lines[1]
    assert "generic fallback" in lines[2]
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       env={k: v for k, v in os.environ.items() if k != "CONVT_LOG"})
    assert "convt:" not in r.stderr


def test_every_kernel_name_has_a_source():
    """Every kernel name the library reports (the string literals "k_..." in
    its sources) maps to its source file in bench.py's table, which decides
    whether a stored counter record still describes the kernel that runs."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    csrc = os.path.join(root, "transposed_convolution_forward_amd", "csrc")
    names = set()
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".cpp")):
            names |= set(re.findall(r'"(k_[a-z0-9_]+)"', open(os.path.join(csrc, f)).read()))
    assert names, "no kernel names found"
    missing = sorted(n for n in names if n not in bench.KERNEL_SOURCES)
    assert not missing, missing
    for n, f in bench.KERNEL_SOURCES.items():
        src = open(os.path.join(csrc, f)).read()
        assert n in src, (n, f)
