"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, each independent of the oracle's own code.

Every pin is a function pin_*(orc) that raises AssertionError on a mismatch.
test_oracle_pins.py runs them on the real oracle; test_oracle_mutants.py runs
them on copies of the oracle with a planted mistake and requires that some pin
fails for every planted mistake.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

from ref_conv import conv_forward, dilate_flip_correlate

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, shape):
    return rng.standard_normal(size=shape).astype(np.float32)


def _forward(orc, x, w, bias=None, add=None, *, groups=1, stride, pad, out_pad, dilation):
    nd = x.ndim - 2
    return orc.forward(ndim=nd, N=x.shape[0], C_in=x.shape[1], C_out=w.shape[1] * groups,
                       groups=groups, in_size=x.shape[2:], K=w.shape[2:], stride=stride, pad=pad,
                       out_pad=out_pad, dilation=dilation, x=x, w=w, bias=bias, add=add)


# Tiny random shapes covering 1D/2D/3D, groups, stride, padding (incl. p > d(K-1)),
# output padding (incl. op >= s) and dilation.
def tiny_cases():
    cases = [
        # ndim, N, Cin, Cout, G, in, K, s, p, op, d
        (1, 2, 3, 4, 1, (7,), (3,), (2,), (1,), (0,), (2,)),
        (1, 1, 4, 6, 2, (5,), (4,), (3,), (2,), (1,), (1,)),
        (1, 2, 2, 2, 1, (6,), (2,), (1,), (0,), (0,), (3,)),
        (1, 1, 2, 3, 1, (4,), (3,), (2,), (5,), (3,), (1,)),   # p > d(K-1), op >= s
        (1, 1, 6, 3, 3, (9,), (5,), (4,), (3,), (2,), (2,)),
        (2, 1, 2, 4, 2, (3, 4), (2, 3), (2, 1), (1, 0), (1, 0), (1, 2)),
        (3, 1, 2, 2, 1, (3, 2, 4), (3, 2, 3), (2, 2, 1), (1, 0, 1), (1, 1, 0), (1, 2, 1)),
        (3, 2, 4, 4, 2, (2, 3, 3), (3, 5, 3), (2, 1, 2), (1, 2, 1), (1, 0, 1), (1, 1, 1)),
        (3, 1, 3, 6, 3, (2, 2, 3), (2, 2, 4), (2, 2, 2), (1, 1, 1), (0, 0, 0), (1, 1, 1)),
    ]
    return cases


def _case_arrays(case, seed):
    nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
    rng = np.random.default_rng(seed)
    x = _rand(rng, (N, Cin) + ins)
    w = _rand(rng, (Cin, Cout // G) + K)
    b = _rand(rng, (Cout,))
    return x, w, b


# ---------------------------------------------------------------------------
def pin_closed_form_pages(orc):
    """E0: output sizes the pages print."""
    for e in _load("closed_form_and_tap_counts.json")["output_sizes"]:
        got = orc.output_size(len(e["in_size"]), e["in_size"], e["K"], e["stride"], e["pad"],
                              e["out_pad"], e["dilation"])
        assert list(got) == e["out_size"], (e["citation"], got)


def pin_worked_examples(orc):
    """E1-E4: symbolic outputs of the pages' worked examples."""
    rng = np.random.default_rng(11)
    for e in _load("worked_examples.json")["examples"]:
        vals = {name: np.float32(rng.standard_normal()) for name in e["x"] + e["w"]}
        x = np.array([[[vals[n] for n in e["x"]]]], dtype=np.float32)
        w = np.array([[[vals[n] for n in e["w"]]]], dtype=np.float32)
        y = _forward(orc, x, w, stride=e["stride"], pad=e["pad"], out_pad=e["out_pad"],
                     dilation=e["dilation"])
        assert list(y.shape[2:]) == e["out_size"], e["id"]
        want = [sum(float(vals[a]) * float(vals[b]) for a, b in terms) for terms in e["y"]]
        np.testing.assert_allclose(y[0, 0], want, rtol=1e-12, atol=1e-12, err_msg=e["id"])
        # an empty term list is an exact zero
        for o, terms in enumerate(e["y"]):
            if not terms:
                assert y[0, 0, o] == 0.0, (e["id"], o)


def pin_numpy_convolve(orc):
    """E5: one channel, stride 1, no padding, no dilation is the full linear
    convolution ("Kimi-K2.6 l1_p72" transcript: stride 1 and padding 0 is a
    full convolution).  Stride s, dilation d, padding 0: full convolution of
    the zero-inserted input with the zero-inserted kernel; output padding
    appends zeros."""
    rng = np.random.default_rng(5)
    for L, K in [(1, 1), (5, 3), (8, 4), (3, 6)]:
        x = _rand(rng, (1, 1, L))
        w = _rand(rng, (1, 1, K))
        y = _forward(orc, x, w, stride=[1], pad=[0], out_pad=[0], dilation=[1])
        np.testing.assert_allclose(y[0, 0], np.convolve(x[0, 0].astype(np.float64),
                                                        w[0, 0].astype(np.float64), "full"),
                                   rtol=1e-12, atol=1e-12)
    for L, K, s, d, op in [(5, 3, 2, 1, 0), (4, 3, 3, 2, 1), (6, 2, 2, 3, 2)]:
        x = _rand(rng, (1, 1, L))
        w = _rand(rng, (1, 1, K))
        xd = np.zeros((L - 1) * s + 1)
        xd[::s] = x[0, 0]
        wd = np.zeros((K - 1) * d + 1)
        wd[::d] = w[0, 0]
        want = np.concatenate([np.convolve(xd, wd, "full"), np.zeros(op)])
        y = _forward(orc, x, w, stride=[s], pad=[0], out_pad=[op], dilation=[d])
        np.testing.assert_allclose(y[0, 0], want, rtol=1e-12, atol=1e-12)


def pin_odd_only(orc):
    """I1: stride 2, padding 1, dilation 2, kernel 3: even outputs equal the
    bias exactly; odd o = 2m-1 gets sum_k W[:, :, k]^T x[:, m-k] over the k with
    0 <= m-k < L_in ("Kimi-K2.6 l1_p79" transcript, the odd-position analysis
    and the boundary count)."""
    rng = np.random.default_rng(7)
    N, Cin, Cout, L = 2, 4, 6, 64
    x = _rand(rng, (N, Cin, L))
    w = _rand(rng, (Cin, Cout, 3))
    b = _rand(rng, (Cout,))
    y = _forward(orc, x, w, b, stride=[2], pad=[1], out_pad=[0], dilation=[2])
    assert y.shape == (N, Cout, 129)
    np.testing.assert_array_equal(y[:, :, 0::2], np.broadcast_to(b.astype(np.float64)[None, :, None],
                                                                 y[:, :, 0::2].shape))
    for m in range(1, L + 1):
        want = b.astype(np.float64)[None, :].repeat(N, 0)
        for k in range(3):
            if 0 <= m - k < L:
                want = want + x[:, :, m - k].astype(np.float64) @ w[:, :, k].astype(np.float64)
        np.testing.assert_allclose(y[:, :, 2 * m - 1], want, rtol=1e-12, atol=1e-12)


def pin_tap_counts(orc):
    """I2: the per-position contribution counts the pages tabulate, both from
    the pair-count routine and from the forward itself (all-ones input and
    weight give, per output, the product of the per-axis counts)."""
    for e in _load("closed_form_and_tap_counts.json")["tap_counts"]:
        c = orc.axis_pair_counts(e["L_in"], e["K"], e["s"], e["p"], e["op"], e["d"])
        assert [int(c[o]) for o in e["positions"]] == e["counts"], e["citation"]
    # forward on ones: the page's 3D axes at reduced input size 4x5x6
    L, K, s, p, op = (4, 5, 6), (3, 5, 7), (2, 2, 2), (1, 2, 3), (1, 1, 1)
    x = np.ones((1, 1) + L, dtype=np.float32)
    w = np.ones((1, 1) + K, dtype=np.float32)
    y = _forward(orc, x, w, stride=s, pad=p, out_pad=op, dilation=(1, 1, 1))
    cnt = [orc.axis_pair_counts(L[a], K[a], s[a], p[a], op[a], 1) for a in range(3)]
    want = cnt[0][:, None, None] * cnt[1][None, :, None] * cnt[2][None, None, :]
    np.testing.assert_array_equal(y[0, 0], want.astype(np.float64))
    # first width counts of the page's table survive the smaller input
    assert list(cnt[2][:8]) == [2, 3, 3, 4, 3, 4, 3, 4]


def pin_adjoint(orc):
    """I4: <convT(x), v> = <x, conv(v)> with bias 0, conv written separately
    in gather form ("Kimi-K2.6 l1_p79" transcript, the adjoint derivation)."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, w, _ = _case_arrays(case, 100 + ci)
        y = _forward(orc, x, w, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        v = np.random.default_rng(200 + ci).standard_normal(size=y.shape)
        lhs = float(np.sum(y * v))
        rhs = float(np.sum(x.astype(np.float64) *
                           conv_forward(v, w, groups=G, in_size=ins, stride=s, pad=p, dilation=d)))
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs)), (case, lhs, rhs)


def pin_dilate_flip_correlate(orc):
    """I5: a second derivation (zero-insert, pad, correlate with the flipped,
    channel-swapped weight) gives the same tensor, bias included."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, w, b = _case_arrays(case, 300 + ci)
        y = _forward(orc, x, w, b, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        want = dilate_flip_correlate(x, w, b, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        assert y.shape == want.shape, case
        np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-11, err_msg=str(case))


def pin_group_decomposition(orc):
    """I6: groups = G is G independent single-group problems on channel slices
    ("Kimi-K2.6 l1_p72" transcript, the per-group channel mapping)."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        if G == 1:
            continue
        x, w, b = _case_arrays(case, 400 + ci)
        y = _forward(orc, x, w, b, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        Cig, Cog = Cin // G, Cout // G
        for g in range(G):
            xs = np.ascontiguousarray(x[:, g * Cig:(g + 1) * Cig])
            ws = np.ascontiguousarray(w[g * Cig:(g + 1) * Cig])
            bs = np.ascontiguousarray(b[g * Cog:(g + 1) * Cog])
            yg = _forward(orc, xs, ws, bs, groups=1, stride=s, pad=p, out_pad=op, dilation=d)
            np.testing.assert_allclose(y[:, g * Cog:(g + 1) * Cog], yg, rtol=1e-12, atol=1e-12)


def pin_epilogue_values(orc):
    """I7: t*hardswish(t) = t^2*clamp(t+3,0,6)/6 ("Kimi-K2.6 l2_p26"
    transcript, its statement of hardswish) at values with closed forms."""
    t = np.array([-4.0, -3.0, -1.0, 0.0, 1.0, 3.0, 6.0, 10.0, -2.5])
    want = np.array([0.0, 0.0, 1.0 / 3.0, 0.0, 2.0 / 3.0, 9.0, 36.0, 100.0, 6.25 * 0.5 / 6.0])
    np.testing.assert_allclose(orc.times_hardswish(t), want, rtol=1e-15, atol=1e-15)


def pin_fused_forward(orc):
    """The fused forward equals the plain forward plus add_input, then the
    epilogue; with add = 0 and t in the linear region it is t^2*(t+3)/6."""
    for ci, case in enumerate(tiny_cases()[:6]):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, w, b = _case_arrays(case, 500 + ci)
        y0 = _forward(orc, x, w, b, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        add = np.random.default_rng(600 + ci).standard_normal(size=y0.shape).astype(np.float32)
        y1 = _forward(orc, x, w, b, add, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        t = y0 + add.astype(np.float64)
        np.testing.assert_allclose(y1, orc.times_hardswish(t), rtol=1e-12, atol=1e-12)
    # second derivation in the region -3 < t < 3 where clamp is the identity
    case = tiny_cases()[0]
    nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
    x, w, b = _case_arrays(case, 700)
    x *= np.float32(0.1)
    t = dilate_flip_correlate(x, w, b, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
    zeros = np.zeros(t.shape, dtype=np.float32)
    y1 = _forward(orc, x, w, b, zeros, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
    assert np.all(np.abs(t) < 3)
    np.testing.assert_allclose(y1, t * t * (t + 3.0) / 6.0, rtol=1e-11, atol=1e-12)


def pin_activation_values(orc):
    """hardswish(t) = t*clamp(t+3,0,6)/6 ("Kimi-K2.6 l2_p26" transcript, its
    statement of hardswish) at values with closed forms; act 0 is the
    identity and act 2 is t*hardswish(t) (the values of pin_epilogue_values)."""
    t = np.array([-4.0, -3.0, -1.0, 0.0, 1.0, 3.0, 6.0, 10.0, -2.5, 1.5])
    want = np.array([0.0, 0.0, -1.0 / 3.0, 0.0, 2.0 / 3.0, 3.0, 6.0, 10.0, -2.5 * 0.5 / 6.0, 1.5 * 4.5 / 6.0])
    np.testing.assert_allclose(orc.activate(t, 1), want, rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(orc.activate(t, 0), t)
    np.testing.assert_allclose(orc.activate(t, 2), t * want, rtol=1e-15, atol=1e-15)


def pin_epilogue_modes(orc):
    """Every epilogue mode is the plain forward (conv + bias), plus add_input
    when given, then the activation, elementwise; in the region -3 < t < 3
    hardswish is t*(t+3)/6, checked against the second derivation."""
    for ci, case in enumerate(tiny_cases()[:5]):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, w, b = _case_arrays(case, 1500 + ci)
        kw = dict(ndim=nd, N=N, C_in=Cin, C_out=Cout, groups=G, in_size=ins, K=K, stride=s, pad=p,
                  out_pad=op, dilation=d, x=x, w=w, bias=b)
        y0 = orc.forward(**kw)
        add = (3 * np.random.default_rng(1600 + ci).standard_normal(size=y0.shape)).astype(np.float32)
        for act in (0, 1, 2):
            np.testing.assert_allclose(orc.forward(act=act, **kw), orc.activate(y0, act), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(orc.forward(add=add, act=act, **kw),
                                       orc.activate(y0 + add.astype(np.float64), act), rtol=1e-12, atol=1e-12)
    case = tiny_cases()[1]
    nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
    x, w, b = _case_arrays(case, 1700)
    x *= np.float32(0.1)
    t = dilate_flip_correlate(x, w, b, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
    assert np.all(np.abs(t) < 3)
    y1 = orc.forward(ndim=nd, N=N, C_in=Cin, C_out=Cout, groups=G, in_size=ins, K=K, stride=s, pad=p,
                     out_pad=op, dilation=d, x=x, w=w, bias=b, act=1)
    np.testing.assert_allclose(y1, t * (t + 3.0) / 6.0, rtol=1e-11, atol=1e-12)


def _to_last(a):
    return np.ascontiguousarray(np.moveaxis(a, 1, -1))


def pin_channels_last(orc):
    """Channels last (x (N, L..., C_in), y and add (N, L..., C_out)) holds the
    same values as channels first, moved: the layout places elements and
    changes no arithmetic.  The one-by-one evaluation agrees in that layout."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, w, b = _case_arrays(case, 1800 + ci)
        kw = dict(ndim=nd, N=N, C_in=Cin, C_out=Cout, groups=G, in_size=ins, K=K, stride=s, pad=p,
                  out_pad=op, dilation=d, w=w, bias=b)
        y0 = orc.forward(x=x, **kw)
        add = np.random.default_rng(1900 + ci).standard_normal(size=y0.shape).astype(np.float32)
        for a, act in ((None, 0), (add, 2), (add, 1)):
            ref = orc.forward(x=x, add=a, act=act, **kw)
            a_l = None if a is None else _to_last(a)
            got = orc.forward(x=_to_last(x), add=a_l, act=act, layout=1, **kw)
            assert got.shape == (N,) + ref.shape[2:] + (Cout,)
            np.testing.assert_array_equal(got, np.moveaxis(ref, 1, -1))
            idx = np.arange(got.size, dtype=np.int64)
            np.testing.assert_allclose(orc.points(idx, x=_to_last(x), add=a_l, act=act, layout=1, **kw),
                                       got.ravel(), rtol=1e-12, atol=1e-12)


def pin_points_match_forward(orc):
    """The one-by-one evaluation (used at full sizes) equals the full forward,
    fused and not, on every element of the tiny cases."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, w, b = _case_arrays(case, 800 + ci)
        kw = dict(ndim=nd, N=N, C_in=Cin, C_out=Cout, groups=G, in_size=ins, K=K, stride=s,
                  pad=p, out_pad=op, dilation=d, x=x, w=w, bias=b)
        y = orc.forward(**kw)
        idx = np.arange(y.size, dtype=np.int64)
        np.testing.assert_allclose(orc.points(idx, **kw), y.ravel(), rtol=1e-12, atol=1e-12)
        add = np.random.default_rng(900 + ci).standard_normal(size=y.shape).astype(np.float32)
        yf = orc.forward(add=add, **kw)
        np.testing.assert_allclose(orc.points(idx, add=add, **kw), yf.ravel(), rtol=1e-12,
                                   atol=1e-12)


def _backward(orc, dy, w, *, groups=1, in_size, stride, pad, out_pad, dilation):
    nd = dy.ndim - 2
    return orc.backward_data(ndim=nd, N=dy.shape[0], C_in=w.shape[0], C_out=dy.shape[1],
                             groups=groups, in_size=in_size, K=w.shape[2:], stride=stride, pad=pad,
                             out_pad=out_pad, dilation=dilation, dy=dy, w=w)


def pin_backward_worked_examples(orc):
    """B1: the input gradient of the pages' worked examples E1-E4 is their
    symbolic matrix read transposed: output o holds terms w_k * x_i, so dx_i
    collects w_k * dy_o over those terms ("Kimi-K2.6 l2_p26" transcript: the
    transposed convolution is C^T, so its adjoint is C)."""
    rng = np.random.default_rng(13)
    for e in _load("worked_examples.json")["examples"]:
        vals = {name: np.float32(rng.standard_normal()) for name in e["w"]}
        dy = rng.standard_normal(size=(1, 1) + tuple(e["out_size"])).astype(np.float32)
        w = np.array([[[vals[n] for n in e["w"]]]], dtype=np.float32)
        dx = _backward(orc, dy, w, in_size=e["in_size"], stride=e["stride"], pad=e["pad"],
                       out_pad=e["out_pad"], dilation=e["dilation"])
        want = np.zeros(len(e["x"]))
        for o, terms in enumerate(e["y"]):
            for wname, xname in terms:
                want[e["x"].index(xname)] += float(vals[wname]) * float(dy[0, 0, o])
        np.testing.assert_allclose(dx[0, 0], want, rtol=1e-12, atol=1e-12, err_msg=e["id"])


def pin_backward_gather(orc):
    """B2: the input gradient equals the strided forward convolution written
    separately in gather form (tests/ref_conv.py) on the tiny shapes."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        _, w, _ = _case_arrays(case, 1100 + ci)
        out = orc.output_size(nd, ins, K, s, p, op, d)
        dy = _rand(np.random.default_rng(1200 + ci), (N, Cout) + out)
        got = _backward(orc, dy, w, groups=G, in_size=ins, stride=s, pad=p, out_pad=op, dilation=d)
        want = conv_forward(dy, w, groups=G, in_size=ins, stride=s, pad=p, dilation=d)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11, err_msg=str(case))


def pin_backward_adjoint(orc):
    """B3: <convT(x), v> = <x, dx(v)> between the oracle's forward (bias 0) and
    its input gradient."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, w, _ = _case_arrays(case, 1300 + ci)
        y = _forward(orc, x, w, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        v = _rand(np.random.default_rng(1400 + ci), y.shape)
        dx = _backward(orc, v, w, groups=G, in_size=ins, stride=s, pad=p, out_pad=op, dilation=d)
        lhs = float(np.sum(y * v.astype(np.float64)))
        rhs = float(np.sum(x.astype(np.float64) * dx))
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs)), (case, lhs, rhs)


def _wgrad(orc, x, dy, K, *, groups=1, stride, pad, out_pad, dilation):
    nd = x.ndim - 2
    return orc.backward_weight(ndim=nd, N=x.shape[0], C_in=x.shape[1], C_out=dy.shape[1], groups=groups,
                               in_size=x.shape[2:], K=K, stride=stride, pad=pad, out_pad=out_pad,
                               dilation=dilation, x=x, dy=dy)


def pin_wgrad_worked_examples(orc):
    """W1: in the pages' worked examples E1-E4 every output element is a list of
    w_k * x_i terms, so the gradient of <y, dy> in w_k collects x_i * dy_o over
    the terms that hold w_k."""
    rng = np.random.default_rng(17)
    for e in _load("worked_examples.json")["examples"]:
        vals = {name: np.float32(rng.standard_normal()) for name in e["x"]}
        x = np.array([[[vals[n] for n in e["x"]]]], dtype=np.float32)
        dy = rng.standard_normal(size=(1, 1) + tuple(e["out_size"])).astype(np.float32)
        dw, db = _wgrad(orc, x, dy, e["K"], stride=e["stride"], pad=e["pad"], out_pad=e["out_pad"],
                        dilation=e["dilation"])
        want = np.zeros(len(e["w"]))
        for o, terms in enumerate(e["y"]):
            for wname, xname in terms:
                want[e["w"].index(wname)] += float(vals[xname]) * float(dy[0, 0, o])
        np.testing.assert_allclose(dw[0, 0], want, rtol=1e-12, atol=1e-12, err_msg=e["id"])
        np.testing.assert_allclose(db, [float(dy.astype(np.float64).sum())], rtol=1e-12, err_msg=e["id"])


def pin_wgrad_adjoint(orc):
    """W2: the forward is linear in w, so <convT(x, u), v> = <u, dw(x, v)> for
    any weight-shaped u; and adding a bias b adds <b, db(v)> to <y, v>."""
    for ci, case in enumerate(tiny_cases()):
        nd, N, Cin, Cout, G, ins, K, s, p, op, d = case
        x, u, b = _case_arrays(case, 1500 + ci)
        y = _forward(orc, x, u, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        v = _rand(np.random.default_rng(1600 + ci), y.shape)
        dw, db = _wgrad(orc, x, v, K, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        lhs = float(np.sum(y * v.astype(np.float64)))
        rhs = float(np.sum(u.astype(np.float64) * dw))
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs)), (case, lhs, rhs)
        yb = _forward(orc, x, u, b, groups=G, stride=s, pad=p, out_pad=op, dilation=d)
        lhs_b = float(np.sum((yb - y) * v.astype(np.float64)))
        rhs_b = float(np.sum(b.astype(np.float64) * db))
        assert abs(lhs_b - rhs_b) <= 1e-9 * (1 + abs(lhs_b)), (case, lhs_b, rhs_b)


ALL_PINS = [pin_closed_form_pages, pin_worked_examples, pin_numpy_convolve, pin_odd_only,
            pin_tap_counts, pin_adjoint, pin_dilate_flip_correlate, pin_group_decomposition,
            pin_epilogue_values, pin_fused_forward, pin_activation_values, pin_epilogue_modes,
            pin_channels_last, pin_points_match_forward,
            pin_backward_worked_examples, pin_backward_gather, pin_backward_adjoint,
            pin_wgrad_worked_examples, pin_wgrad_adjoint]
