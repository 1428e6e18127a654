"""Shared test helpers: ulp metrics, tolerances and an independent fp64 formulation."""
from __future__ import annotations

import numpy as np
import torch


def ordered(t: torch.Tensor) -> torch.Tensor:
    """Map floats to integers that are ordered like the values (+0 == -0), as int64."""
    if t.dtype in (torch.float16, torch.bfloat16):
        b = t.contiguous().view(torch.int16).to(torch.int64) & 0xFFFF
        mag = b & 0x7FFF
        return torch.where(b >= 0x8000, -mag, mag)
    if t.dtype == torch.float32:
        b = t.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
        mag = b & 0x7FFFFFFF
        return torch.where(b >= 0x80000000, -mag, mag)
    raise TypeError(t.dtype)


def ulp_dist(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    assert a.dtype == b.dtype and a.shape == b.shape
    return (ordered(a) - ordered(b)).abs()


def ulp_of(x: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """Spacing of T numbers at |x| (x given as float64)."""
    x = x.abs().to(torch.float64)
    mant = {torch.float16: 10, torch.bfloat16: 7, torch.float32: 23}[dtype]
    emin = {torch.float16: -14, torch.bfloat16: -126, torch.float32: -126}[dtype]
    e = torch.floor(torch.log2(torch.clamp(x, min=2.0 ** emin)))
    return torch.pow(2.0, e - mant)


def ref64(streams, ns, wd, wu, wi, prev_out=None, prev_gate=None, *, num_branches, epsilon,
          reduction_scale, silu_alpha, gate_div, gate_mul):
    """The block from the pages' "Schema summary" in float64 numpy, no rounding,
    written as whole-array operations (independent of the oracle's loops).
    Returns pre, post, S and the magnitudes feeding the last rounding."""
    C = num_branches
    X = streams.double().numpy()
    M, K = X.shape
    H = K // C
    S = X.reshape(M, C, H).copy()
    if prev_out is not None:
        S = S + prev_gate.double().numpy()[:, :, None] * prev_out.double().numpy()[:, None, :]
    rms = np.sqrt((S ** 2).mean(axis=2, keepdims=True) + epsilon)
    hn = (S / rms) * ns.double().numpy().reshape(1, C, H)
    hnf = hn.reshape(M, K)
    d = hnf @ wd.double().numpy()
    hid = d / (1.0 + np.exp(-silu_alpha * d))
    g = 1.0 / (1.0 + np.exp(-(hid @ wu.double().numpy())))
    prod = hn * g.reshape(M, C, H)
    pre = reduction_scale * prod.sum(axis=1)
    pre_mag = abs(reduction_scale) * np.abs(prod).sum(axis=1)
    post = gate_mul / (1.0 + np.exp(-(hnf @ wi.double().numpy()) / gate_div))
    return pre, post, S.reshape(M, K), pre_mag
