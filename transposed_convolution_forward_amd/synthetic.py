"""Seeded synthetic inputs for the transposed-convolution workloads.

This module is shared by the HIP path's tests and bench and by the CPU oracle's
tests.  It holds only workload descriptions (shapes and layer parameters) and
random-number draws.  It holds none of the convolution's arithmetic: no output
shape, no index mapping, no contraction.  Each side computes those on its own.

Distributions: x and add_input ~ N(0, 1); weight and bias ~ U(-B, +B) with
B = 1/sqrt((C_in/groups) * prod(K)) (the default initialisation bound of a
transposed-convolution layer, applied to the workload's shape).  Each tensor
draws from its own stream, PCG64(SeedSequence([seed, workload_id, tensor_id])),
tensor ids x=0, w=1, bias=2, add_input=3.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

TENSOR_X, TENSOR_W, TENSOR_BIAS, TENSOR_ADD = 0, 1, 2, 3
TENSOR_DY = 4  # the output gradient fed to the input-gradient pass


@dataclasses.dataclass(frozen=True)
class Workload:
    """One transposed-convolution layer and batch shape (all per-axis tuples)."""
    name: str
    ndim: int
    N: int
    C_in: int
    C_out: int
    groups: int
    in_size: Tuple[int, ...]
    K: Tuple[int, ...]
    stride: Tuple[int, ...]
    pad: Tuple[int, ...]
    out_pad: Tuple[int, ...]
    dilation: Tuple[int, ...]
    bias: bool
    fused: bool  # conv + bias + add_input, then t * hardswish(t)
    wid: int = 0  # workload id, part of the seed sequence

    def params(self):
        return dict(ndim=self.ndim, N=self.N, C_in=self.C_in, C_out=self.C_out,
                    groups=self.groups, in_size=self.in_size, K=self.K,
                    stride=self.stride, pad=self.pad, out_pad=self.out_pad,
                    dilation=self.dilation)

    def x_shape(self):
        return (self.N, self.C_in) + tuple(self.in_size)

    def w_shape(self):
        return (self.C_in, self.C_out // self.groups) + tuple(self.K)

    def init_bound(self) -> float:
        return 1.0 / math.sqrt((self.C_in // self.groups) * math.prod(self.K))

    def with_batch(self, N: int) -> "Workload":
        return dataclasses.replace(self, N=N)


def _rng(seed: int, wid: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, tensor_id])))


def normal(shape: Sequence[int], seed: int, wid: int, tensor_id: int) -> np.ndarray:
    return _rng(seed, wid, tensor_id).standard_normal(size=tuple(shape), dtype=np.float32)


def uniform(shape: Sequence[int], bound: float, seed: int, wid: int, tensor_id: int) -> np.ndarray:
    u = _rng(seed, wid, tensor_id).random(size=tuple(shape), dtype=np.float32)
    return ((u * np.float32(2.0) - np.float32(1.0)) * np.float32(bound)).astype(np.float32)


def small_integers(shape: Sequence[int], bound: int, seed: int, wid: int, tensor_id: int) -> np.ndarray:
    """Integers drawn uniformly from [-bound, bound], as float32.  Sums of
    products of such values stay exact in fp32 while below 2^24, so a result
    computed from them does not depend on the order of its additions."""
    v = _rng(seed, wid, tensor_id).integers(-bound, bound + 1, size=tuple(shape))
    return v.astype(np.float32)


def make_inputs(wl: Workload, seed: int = 0, out_shape: Optional[Sequence[int]] = None):
    """Return dict(x, w, bias|None, add|None) of float32 arrays.

    add_input needs the output shape, which this module does not compute: the
    caller passes it (each side derives it on its own).
    """
    B = wl.init_bound()
    d = {
        "x": normal(wl.x_shape(), seed, wl.wid, TENSOR_X),
        "w": uniform(wl.w_shape(), B, seed, wl.wid, TENSOR_W),
        "bias": uniform((wl.C_out,), B, seed, wl.wid, TENSOR_BIAS) if wl.bias else None,
        "add": None,
    }
    if wl.fused:
        if out_shape is None:
            raise ValueError("fused workload needs out_shape for add_input")
        d["add"] = normal(tuple(out_shape), seed, wl.wid, TENSOR_ADD)
    return d


def make_grad_output(wl: Workload, seed: int, out_shape: Sequence[int]):
    """dy ~ N(0, 1) in the forward output's shape, for the input gradient."""
    return normal(tuple(out_shape), seed, wl.wid, TENSOR_DY)


# The five workloads: a tiny 1D case, the long-sequence 1D case, a grouped
# asymmetric 3D case, the fused 3D case and a channel-heavy 3D case.
TINY_1D = Workload("convT1d_tiny_N2_C4to6_L64_K3_s2_p1_d2", 1, 2, 4, 6, 1, (64,), (3,), (2,), (1,),
                   (0,), (2,), True, False, wid=1)
LONG_1D = Workload("convT1d_N16_C32to64_L131072_K3_s2_p1_d2", 1, 16, 32, 64, 1, (131072,), (3,),
                   (2,), (1,), (0,), (2,), False, False, wid=2)
GROUPED_3D = Workload("convT3d_N8_C32to32_g4_K3x5x7_s2x1x2_in16x32x32", 3, 8, 32, 32, 4,
                      (16, 32, 32), (3, 5, 7), (2, 1, 2), (1, 2, 3), (1, 0, 1), (1, 1, 1), True,
                      False, wid=3)
FUSED_3D = Workload("convT3d_add_hswish_N128_C32to64_K3_s2_in16", 3, 128, 32, 64, 1, (16, 16, 16),
                    (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), (1, 1, 1), True, True, wid=4)
HEAVY_3D = Workload("convT3d_N8_C128to64_K4_s2_in32", 3, 8, 128, 64, 1, (32, 32, 32), (4, 4, 4),
                    (2, 2, 2), (1, 1, 1), (0, 0, 0), (1, 1, 1), True, False, wid=5)

WORKLOADS = [TINY_1D, LONG_1D, GROUPED_3D, FUSED_3D, HEAVY_3D]
BY_NAME = {w.name: w for w in WORKLOADS}
