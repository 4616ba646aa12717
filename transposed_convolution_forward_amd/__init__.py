"""Transposed-convolution forward on AMD MI355X: Python binding of libconvt.so.

The binding only marshals arguments to the C ABI declared in include/convt.h
(same function names).  Every step of the computation runs in the library's
HIP kernels; torch supplies device memory and the current stream.  There is no
fallback: if libconvt.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libconvt.so")

CONVT_OK, CONVT_ERR_INVALID_ARG, CONVT_ERR_UNSUPPORTED, CONVT_ERR_HIP, CONVT_ERR_NOMEM = range(5)
PATHS = {"auto": 0, "generic": 1, "stream1d": 2, "igemm3d": 3}
ACTIVATIONS = {"none": 0, "hardswish": 1, "x_hardswish": 2}  # convt_activation
LAYOUTS = {"channels_first": 0, "channels_last": 1}  # convt_layout
LAYOUT_NAMES = {v: k for k, v in LAYOUTS.items()}
PATH_NAMES = {v: k for k, v in PATHS.items()}

# Every symbol include/convt.h declares.
EXPORTS = ("convt_plan_create", "convt_plan_output_size", "convt_forward",
           "convt_forward_add_hswish", "convt_forward_epilogue", "convt_backward_data", "convt_backward_weight",
           "convt_plan_destroy", "convt_status_string",
           "convt_plan_set_path", "convt_plan_get_path", "convt_plan_set_layout", "convt_plan_get_layout",
           "convt_plan_describe")

_lib_handle = None
_i64p = ctypes.POINTER(ctypes.c_int64)


class ConvtError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {convt_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libconvt.so (once).  Raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m "
                           "transposed_convolution_forward_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    L.convt_plan_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int] + [ctypes.c_int64] * 4 + [_i64p] * 6
    L.convt_plan_create.restype = ctypes.c_int
    L.convt_plan_output_size.argtypes = [vp, _i64p]
    L.convt_plan_output_size.restype = ctypes.c_int
    L.convt_forward.argtypes = [vp, vp, vp, vp, vp, vp]
    L.convt_forward.restype = ctypes.c_int
    L.convt_forward_add_hswish.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.convt_forward_add_hswish.restype = ctypes.c_int
    L.convt_forward_epilogue.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp]
    L.convt_forward_epilogue.restype = ctypes.c_int
    L.convt_backward_data.argtypes = [vp, vp, vp, vp, vp]
    L.convt_backward_data.restype = ctypes.c_int
    L.convt_backward_weight.argtypes = [vp, vp, vp, vp, vp, vp]
    L.convt_backward_weight.restype = ctypes.c_int
    L.convt_plan_destroy.argtypes = [vp]
    L.convt_plan_destroy.restype = None
    L.convt_status_string.argtypes = [ctypes.c_int]
    L.convt_status_string.restype = ctypes.c_char_p
    L.convt_plan_set_path.argtypes = [vp, ctypes.c_int]
    L.convt_plan_set_path.restype = ctypes.c_int
    L.convt_plan_get_path.argtypes = [vp]
    L.convt_plan_get_path.restype = ctypes.c_int
    L.convt_plan_set_layout.argtypes = [vp, ctypes.c_int]
    L.convt_plan_set_layout.restype = ctypes.c_int
    L.convt_plan_get_layout.argtypes = [vp]
    L.convt_plan_get_layout.restype = ctypes.c_int
    L.convt_plan_describe.argtypes = [vp, ctypes.c_char_p, ctypes.c_int64]
    L.convt_plan_describe.restype = ctypes.c_int64
    _lib_handle = L
    return L


def _arr(v: Sequence[int]):
    return (ctypes.c_int64 * len(v))(*[int(a) for a in v])


class Plan:
    """Owns one convt_plan*; destroyed with the object."""

    def __init__(self, ndim: int, N: int, C_in: int, C_out: int, groups: int,
                 in_size: Sequence[int], K: Sequence[int], stride: Sequence[int],
                 pad: Sequence[int], out_pad: Sequence[int], dilation: Sequence[int]):
        L = lib()
        for name, v in (("in_size", in_size), ("K", K), ("stride", stride), ("pad", pad),
                        ("out_pad", out_pad), ("dilation", dilation)):
            if len(v) != ndim:
                raise ValueError(f"{name} needs {ndim} entries")
        h = ctypes.c_void_p()
        st = L.convt_plan_create(ctypes.byref(h), int(ndim), int(N), int(C_in), int(C_out),
                                 int(groups), _arr(in_size), _arr(K), _arr(stride), _arr(pad),
                                 _arr(out_pad), _arr(dilation))
        if st != CONVT_OK:
            raise ConvtError(st, "convt_plan_create")
        self._h = h
        self.layout = "channels_first"
        self.ndim, self.N, self.C_in, self.C_out, self.groups = ndim, N, C_in, C_out, groups
        self.in_size, self.K = tuple(in_size), tuple(K)
        out = (ctypes.c_int64 * ndim)()
        st = L.convt_plan_output_size(h, out)
        if st != CONVT_OK:
            raise ConvtError(st, "convt_plan_output_size")
        self.out_size = tuple(int(v) for v in out)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib_handle is not None:
            _lib_handle.convt_plan_destroy(h)
            self._h = None

    def x_shape(self):
        if self.layout == "channels_last":
            return (self.N,) + self.in_size + (self.C_in,)
        return (self.N, self.C_in) + self.in_size

    def w_shape(self):
        return (self.C_in, self.C_out // self.groups) + self.K

    def y_shape(self):
        if self.layout == "channels_last":
            return (self.N,) + self.out_size + (self.C_out,)
        return (self.N, self.C_out) + self.out_size


def _dev_ptr(t, shape, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# --- the C ABI, same names ------------------------------------------------
def convt_plan_create(ndim, N, C_in, C_out, groups, in_size, K, stride, pad, out_pad,
                      dilation) -> Plan:
    return Plan(ndim, N, C_in, C_out, groups, in_size, K, stride, pad, out_pad, dilation)


def convt_plan_output_size(plan: Plan):
    return plan.out_size


def convt_forward(plan: Plan, x, w, bias=None, y=None, stream=None):
    """y = conv_transpose(x, w) + bias on the current (or given) stream."""
    import torch
    if y is None:
        y = torch.empty(plan.y_shape(), dtype=torch.float32, device=x.device)
    args = (_dev_ptr(x, plan.x_shape(), "x"), _dev_ptr(w, plan.w_shape(), "w"),
            None if bias is None else _dev_ptr(bias, (plan.C_out,), "bias"),
            _dev_ptr(y, plan.y_shape(), "y"))
    st = lib().convt_forward(plan.handle, *args, _stream_ptr(stream))
    if st != CONVT_OK:
        raise ConvtError(st, "convt_forward")
    return y


def convt_forward_add_hswish(plan: Plan, x, w, bias, add_input, y=None, stream=None):
    """t = conv_transpose(x, w) + bias + add_input; y = t * hardswish(t)."""
    import torch
    if y is None:
        y = torch.empty(plan.y_shape(), dtype=torch.float32, device=x.device)
    args = (_dev_ptr(x, plan.x_shape(), "x"), _dev_ptr(w, plan.w_shape(), "w"),
            None if bias is None else _dev_ptr(bias, (plan.C_out,), "bias"),
            _dev_ptr(add_input, plan.y_shape(), "add_input"), _dev_ptr(y, plan.y_shape(), "y"))
    st = lib().convt_forward_add_hswish(plan.handle, *args, _stream_ptr(stream))
    if st != CONVT_OK:
        raise ConvtError(st, "convt_forward_add_hswish")
    return y


def convt_forward_epilogue(plan: Plan, x, w, bias=None, add_input=None, activation="none", y=None,
                           stream=None):
    """t = conv_transpose(x, w) + bias [+ add_input]; y = t, hardswish(t) or
    t * hardswish(t) (activation "none", "hardswish" or "x_hardswish", or the
    enum's integer)."""
    import torch
    act = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
    if y is None:
        y = torch.empty(plan.y_shape(), dtype=torch.float32, device=x.device)
    args = (_dev_ptr(x, plan.x_shape(), "x"), _dev_ptr(w, plan.w_shape(), "w"),
            None if bias is None else _dev_ptr(bias, (plan.C_out,), "bias"),
            None if add_input is None else _dev_ptr(add_input, plan.y_shape(), "add_input"))
    st = lib().convt_forward_epilogue(plan.handle, *args, act, _dev_ptr(y, plan.y_shape(), "y"),
                                      _stream_ptr(stream))
    if st != CONVT_OK:
        raise ConvtError(st, "convt_forward_epilogue")
    return y


def convt_backward_data(plan: Plan, dy, w, dx=None, stream=None):
    """dx = the input gradient of the forward's linear part, applied to dy."""
    import torch
    if dx is None:
        dx = torch.empty(plan.x_shape(), dtype=torch.float32, device=dy.device)
    args = (_dev_ptr(dy, plan.y_shape(), "dy"), _dev_ptr(w, plan.w_shape(), "w"),
            _dev_ptr(dx, plan.x_shape(), "dx"))
    st = lib().convt_backward_data(plan.handle, *args, _stream_ptr(stream))
    if st != CONVT_OK:
        raise ConvtError(st, "convt_backward_data")
    return dx


def convt_backward_weight(plan: Plan, x, dy, dw=None, db=None, with_bias: bool = True, stream=None):
    """(dw, db): weight and bias gradients for the output gradient dy (db is
    None when with_bias is False and no db tensor is given)."""
    import torch
    if dw is None:
        dw = torch.empty(plan.w_shape(), dtype=torch.float32, device=x.device)
    if db is None and with_bias:
        db = torch.empty((plan.C_out,), dtype=torch.float32, device=x.device)
    args = (_dev_ptr(x, plan.x_shape(), "x"), _dev_ptr(dy, plan.y_shape(), "dy"),
            _dev_ptr(dw, plan.w_shape(), "dw"), None if db is None else _dev_ptr(db, (plan.C_out,), "db"))
    st = lib().convt_backward_weight(plan.handle, *args, _stream_ptr(stream))
    if st != CONVT_OK:
        raise ConvtError(st, "convt_backward_weight")
    return dw, db


def convt_plan_destroy(plan: Plan) -> None:
    h = plan._h
    if h is not None:
        lib().convt_plan_destroy(h)
        plan._h = None


def convt_status_string(status: int) -> str:
    return lib().convt_status_string(int(status)).decode()


def convt_plan_set_path(plan: Plan, path: str) -> None:
    st = lib().convt_plan_set_path(plan.handle, PATHS[path])
    if st != CONVT_OK:
        raise ConvtError(st, f"convt_plan_set_path({path})")


def convt_plan_get_path(plan: Plan) -> str:
    return PATH_NAMES[lib().convt_plan_get_path(plan.handle)]


def convt_plan_set_layout(plan: Plan, layout: str) -> None:
    """"channels_first" (N, C, L...) or "channels_last" (N, L..., C) for x, y
    and add_input; the tensor shapes the calls expect follow."""
    st = lib().convt_plan_set_layout(plan.handle, LAYOUTS[layout])
    if st != CONVT_OK:
        raise ConvtError(st, f"convt_plan_set_layout({layout})")
    plan.layout = layout


def convt_plan_get_layout(plan: Plan) -> str:
    return LAYOUT_NAMES[lib().convt_plan_get_layout(plan.handle)]


def convt_plan_describe(plan: Plan) -> str:
    n = lib().convt_plan_describe(plan.handle, None, 0)
    buf = ctypes.create_string_buffer(int(n) + 1)
    lib().convt_plan_describe(plan.handle, buf, int(n) + 1)
    return buf.value.decode()


def plan_for(wl, layout: str = "channels_first") -> Plan:
    """Plan for a synthetic.Workload description, in the given layout."""
    p = Plan(wl.ndim, wl.N, wl.C_in, wl.C_out, wl.groups, wl.in_size, wl.K, wl.stride, wl.pad,
             wl.out_pad, wl.dilation)
    if layout != "channels_first":
        convt_plan_set_layout(p, layout)
    return p
