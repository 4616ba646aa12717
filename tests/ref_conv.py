"""Independent numpy formulations used to pin the oracle (tests only).

Nothing here is shared with the oracle (oracle/convt_oracle.c) or with the HIP
library; each function is written from its own definition.

* conv_forward: the strided, padded, dilated forward convolution whose adjoint
  is the transposed convolution.  "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d,
  dilation 2), the adjoint derivation <y, u> = <conv(y), z>; "Kimi-K2.6 l2_p26"
  transcript, the C^T example (conv matrix C, transposed).
  Gather form: out[n, ci, i] = sum_{co_l, k} w[ci, co_l, k] * v[n, g*Cog+co_l, i*s - p + k*d],
  zero where the index leaves [0, L_v).

* dilate_flip_correlate: zero-insert the input by the stride, pad d*(K-1)-p on
  the low side and d*(K-1)-p+out_pad on the high side (negative pad = crop), and
  correlate with the spatially flipped weight taken as (C_out, C_in) per group,
  dilated by d.  "Kimi-K2.6 l1_p72" transcript (ConvTranspose3d), the
  "effective padding" derivation that settles on flipping the kernel;
  "Kimi-K2.6 l2_p26" transcript, the zero-inserted-input emulation.
"""
from __future__ import annotations

import itertools

import numpy as np


def _axes_lists(ndim, *per_axis):
    return [tuple(int(v) for v in a) for a in per_axis]


def conv_forward(v, w, *, groups, in_size, stride, pad, dilation):
    """Forward strided convolution from the output space back to the input
    space: v has shape (N, C_out, *L_v), result (N, C_in, *in_size), float64."""
    v = np.asarray(v, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, C_out = v.shape[:2]
    C_in = w.shape[0]
    Cog = w.shape[1]
    Cig = C_in // groups
    nd = len(in_size)
    L_v = v.shape[2:]
    K = w.shape[2:]
    out = np.zeros((N, C_in) + tuple(in_size), dtype=np.float64)
    for g in range(groups):
        vg = v[:, g * Cog:(g + 1) * Cog]                # (N, Cog, *L_v)
        wg = w[g * Cig:(g + 1) * Cig]                   # (Cig, Cog, *K)
        for kk in itertools.product(*[range(k) for k in K]):
            # per axis: source index i*s - p + k*d for every i in [0, in_size)
            idx, ok = [], []
            for a in range(nd):
                src = np.arange(in_size[a]) * stride[a] - pad[a] + kk[a] * dilation[a]
                ok.append((src >= 0) & (src < L_v[a]))
                idx.append(np.clip(src, 0, L_v[a] - 1))
            grid = np.ix_(*idx)
            mask = np.ones(tuple(in_size), dtype=bool)
            for a in range(nd):
                shp = [1] * nd
                shp[a] = in_size[a]
                mask = mask & ok[a].reshape(shp)
            gathered = vg[(slice(None), slice(None)) + grid]          # (N, Cog, *in_size)
            gathered = gathered * mask
            wk = wg[(slice(None), slice(None)) + kk]                  # (Cig, Cog)
            out[:, g * Cig:(g + 1) * Cig] += np.einsum("ncs,ic->nis",
                                                       gathered.reshape(N, Cog, -1),
                                                       wk).reshape((N, Cig) + tuple(in_size))
    return out


def dilate_flip_correlate(x, w, bias=None, *, groups, stride, pad, out_pad, dilation):
    """Transposed convolution as: zero-insert, pad, correlate with the flipped,
    channel-swapped weight.  Returns float64 (N, C_out, *L_out)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, C_in = x.shape[:2]
    L_in = x.shape[2:]
    nd = len(L_in)
    Cog = w.shape[1]
    C_out = Cog * groups
    Cig = C_in // groups
    K = w.shape[2:]
    # 1. zero insertion: x_d[j] = x[i] at j = i*s
    L_d = [(L_in[a] - 1) * stride[a] + 1 for a in range(nd)]
    xd = np.zeros((N, C_in) + tuple(L_d))
    xd[(slice(None), slice(None)) + tuple(slice(0, L_d[a], stride[a]) for a in range(nd))] = x
    # 2. pad (or crop) each side
    lo = [dilation[a] * (K[a] - 1) - pad[a] for a in range(nd)]
    hi = [dilation[a] * (K[a] - 1) - pad[a] + out_pad[a] for a in range(nd)]
    L_p = [L_d[a] + lo[a] + hi[a] for a in range(nd)]
    xp = np.zeros((N, C_in) + tuple(max(l, 0) for l in L_p))
    src_sl, dst_sl = [], []
    for a in range(nd):
        s0 = max(0, -lo[a])                  # first x_d index kept
        d0 = max(0, lo[a])                   # where it lands
        n = min(L_d[a] - s0, L_p[a] - d0)
        src_sl.append(slice(s0, s0 + max(n, 0)))
        dst_sl.append(slice(d0, d0 + max(n, 0)))
    xp[(slice(None), slice(None)) + tuple(dst_sl)] = xd[(slice(None), slice(None)) + tuple(src_sl)]
    # 3. correlate with flipped weight, dilated
    L_out = [L_p[a] - dilation[a] * (K[a] - 1) for a in range(nd)]
    y = np.zeros((N, C_out) + tuple(L_out))
    wf = w[(slice(None), slice(None)) + tuple(slice(None, None, -1) for _ in range(nd))]
    for g in range(groups):
        xg = xp[:, g * Cig:(g + 1) * Cig]
        wg = wf[g * Cig:(g + 1) * Cig]                     # (Cig, Cog, *K) flipped
        for kk in itertools.product(*[range(k) for k in K]):
            win = xg[(slice(None), slice(None)) + tuple(
                slice(kk[a] * dilation[a], kk[a] * dilation[a] + L_out[a]) for a in range(nd))]
            wk = wg[(slice(None), slice(None)) + kk]          # (Cig, Cog)
            y[:, g * Cog:(g + 1) * Cog] += np.einsum("nis,io->nos", win.reshape(N, Cig, -1),
                                                     wk).reshape((N, Cog) + tuple(L_out))
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64).reshape((1, C_out) + (1,) * nd)
    return y
