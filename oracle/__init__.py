"""Python handle on the CPU oracle (oracle/convt_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg use it.  The product package never imports it.

The oracle is the direct scatter definition of the transposed convolution in
fp64 (see the header of convt_oracle.c for the passages it follows).  This
wrapper only marshals numpy arrays through ctypes; it adds no arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "convt_oracle.c")
LIB = os.path.join(HERE, "liboracle_convt.so")

_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(src: str = SRC, out: str = LIB, extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with the host C compiler (plain C, pthreads)."""
    cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
           "-Wall", "-Wextra", *extra_flags, "-o", out + ".tmp", src, "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _arr(a: Sequence[int]):
    return (ctypes.c_int64 * len(a))(*[int(v) for v in a])


def _f32(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_f32p)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str = LIB):
        if path == LIB and (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build()
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_output_size.argtypes = [ctypes.c_int] + [_i64p] * 7
        lib.oracle_output_size.restype = ctypes.c_int
        conv_args = [ctypes.c_int] + [ctypes.c_int64] * 4 + [_i64p] * 6 + [_f32p] * 4
        lib.oracle_convt_forward.argtypes = conv_args + [_f64p, ctypes.c_int]
        lib.oracle_convt_forward.restype = ctypes.c_int
        lib.oracle_convt_points.argtypes = conv_args + [_i64p, ctypes.c_int64, _f64p]
        lib.oracle_convt_points.restype = ctypes.c_int
        lib.oracle_convt_forward_ex.argtypes = conv_args + [ctypes.c_int, ctypes.c_int, _f64p, ctypes.c_int]
        lib.oracle_convt_forward_ex.restype = ctypes.c_int
        lib.oracle_convt_points_ex.argtypes = conv_args + [ctypes.c_int, ctypes.c_int, _i64p, ctypes.c_int64,
                                                           _f64p]
        lib.oracle_convt_points_ex.restype = ctypes.c_int
        lib.oracle_activate.argtypes = [_f64p, _f64p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_activate.restype = None
        lib.oracle_axis_pair_counts.argtypes = [ctypes.c_int64] * 6 + [_i64p]
        lib.oracle_axis_pair_counts.restype = ctypes.c_int
        lib.oracle_times_hardswish.argtypes = [_f64p, _f64p, ctypes.c_int64]
        lib.oracle_times_hardswish.restype = None
        lib.oracle_convt_backward_data.argtypes = ([ctypes.c_int] + [ctypes.c_int64] * 4 + [_i64p] * 6 +
                                                   [_f32p] * 2 + [_f64p, ctypes.c_int])
        lib.oracle_convt_backward_data.restype = ctypes.c_int
        lib.oracle_convt_backward_weight.argtypes = ([ctypes.c_int] + [ctypes.c_int64] * 4 + [_i64p] * 6 +
                                                     [_f32p] * 2 + [_f64p, _f64p, ctypes.c_int])
        lib.oracle_convt_backward_weight.restype = ctypes.c_int
        self.lib = lib

    # -- shapes -----------------------------------------------------------
    def output_size(self, ndim, in_size, K, stride, pad, out_pad, dilation):
        out = (ctypes.c_int64 * ndim)()
        rc = self.lib.oracle_output_size(ndim, _arr(in_size), _arr(K), _arr(stride), _arr(pad),
                                         _arr(out_pad), _arr(dilation), out)
        if rc:
            raise ValueError("bad arguments")
        return tuple(int(v) for v in out)

    def axis_pair_counts(self, L_in, K, s, p, op, d) -> np.ndarray:
        (L_out,) = self.output_size(1, [L_in], [K], [s], [p], [op], [d])
        if L_out < 1:
            raise ValueError("L_out < 1")
        out = np.zeros(L_out, dtype=np.int64)
        rc = self.lib.oracle_axis_pair_counts(L_in, K, s, p, op, d, out.ctypes.data_as(_i64p))
        if rc:
            raise ValueError("bad arguments")
        return out

    # -- values -----------------------------------------------------------
    def forward(self, *, ndim, N, C_in, C_out, groups, in_size, K, stride, pad, out_pad, dilation,
                x, w, bias=None, add=None, act=None, layout=0, nthreads: int = 0) -> np.ndarray:
        """Whole output as float64, shape (N, C_out, *L_out) for layout 0
        (channels first) or (N, *L_out, C_out) for layout 1 (channels last),
        x and add in the same layout.  act: 0 none, 1 hardswish, 2 t *
        hardswish(t); None means 2 with add and 0 without (the two forwards
        of the pages)."""
        out_size = self.output_size(ndim, in_size, K, stride, pad, out_pad, dilation)
        if act is None:
            act = 2 if add is not None else 0
        shape = (N,) + out_size + (C_out,) if layout else (N, C_out) + out_size
        y = np.empty(shape, dtype=np.float64)
        rc = self.lib.oracle_convt_forward_ex(
            ndim, N, C_in, C_out, groups, _arr(in_size), _arr(K), _arr(stride), _arr(pad),
            _arr(out_pad), _arr(dilation), _f32(x), _f32(w), _f32(bias), _f32(add), int(act), int(layout),
            y.ctypes.data_as(_f64p), int(nthreads))
        if rc:
            raise ValueError("bad arguments")
        return y

    def points(self, idx: np.ndarray, *, ndim, N, C_in, C_out, groups, in_size, K, stride, pad,
               out_pad, dilation, x, w, bias=None, add=None, act=None, layout=0) -> np.ndarray:
        """Output values at flat indices idx (of the layout's output shape),
        computed one by one, float64; act and layout as forward()."""
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        out = np.empty(idx.shape, dtype=np.float64)
        if act is None:
            act = 2 if add is not None else 0
        rc = self.lib.oracle_convt_points_ex(
            ndim, N, C_in, C_out, groups, _arr(in_size), _arr(K), _arr(stride), _arr(pad),
            _arr(out_pad), _arr(dilation), _f32(x), _f32(w), _f32(bias), _f32(add), int(act), int(layout),
            idx.ctypes.data_as(_i64p), idx.size, out.ctypes.data_as(_f64p))
        if rc:
            raise ValueError("bad arguments")
        return out

    def backward_data(self, *, ndim, N, C_in, C_out, groups, in_size, K, stride, pad, out_pad, dilation,
                      dy, w, nthreads: int = 0) -> np.ndarray:
        """Input gradient dx (adjoint of the forward's linear part) as float64,
        shape (N, C_in, *in_size); dy has the forward output's shape."""
        dx = np.empty((N, C_in) + tuple(int(v) for v in in_size), dtype=np.float64)
        rc = self.lib.oracle_convt_backward_data(
            ndim, N, C_in, C_out, groups, _arr(in_size), _arr(K), _arr(stride), _arr(pad),
            _arr(out_pad), _arr(dilation), _f32(dy), _f32(w), dx.ctypes.data_as(_f64p), int(nthreads))
        if rc:
            raise ValueError("bad arguments")
        return dx

    def backward_weight(self, *, ndim, N, C_in, C_out, groups, in_size, K, stride, pad, out_pad,
                        dilation, x, dy, nthreads: int = 0):
        """(dw, db) as float64: dw (C_in, C_out/groups, *K), db (C_out,)."""
        dw = np.empty((C_in, C_out // groups) + tuple(int(v) for v in K), dtype=np.float64)
        db = np.empty((C_out,), dtype=np.float64)
        rc = self.lib.oracle_convt_backward_weight(
            ndim, N, C_in, C_out, groups, _arr(in_size), _arr(K), _arr(stride), _arr(pad),
            _arr(out_pad), _arr(dilation), _f32(x), _f32(dy), dw.ctypes.data_as(_f64p),
            db.ctypes.data_as(_f64p), int(nthreads))
        if rc:
            raise ValueError("bad arguments")
        return dw, db

    def activate(self, t: np.ndarray, act: int) -> np.ndarray:
        t = np.ascontiguousarray(t, dtype=np.float64)
        out = np.empty_like(t)
        self.lib.oracle_activate(t.ctypes.data_as(_f64p), out.ctypes.data_as(_f64p), t.size, int(act))
        return out

    def times_hardswish(self, t: np.ndarray) -> np.ndarray:
        t = np.ascontiguousarray(t, dtype=np.float64)
        out = np.empty_like(t)
        self.lib.oracle_times_hardswish(t.ctypes.data_as(_f64p), out.ctypes.data_as(_f64p), t.size)
        return out


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
