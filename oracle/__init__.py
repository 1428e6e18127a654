"""Python access to the CPU oracle (``hclrmix_oracle.c``).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg use it; the HIP library never does. Arguments are CPU torch
tensors of element type T (contiguous, row-major); results come back the same
way. See ``hclrmix_oracle.c`` for what is computed and the readings taken.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhclrmix_oracle.so")

DTYPE_CODE = {torch.float32: 1, torch.float16: 10, torch.bfloat16: 16}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run oracle/build.py first")
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, F, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        D = ctypes.c_double
        common = [I, I64, I64, I64, I64] + [P] * 10
        lib.hclrmix_oracle_run.restype = I
        lib.hclrmix_oracle_run.argtypes = common + [F] * 5 + [I]
        lib.hclrmix_oracle_run_mag.restype = I
        lib.hclrmix_oracle_run_mag.argtypes = common + [F] * 5 + [I, P]
        lib.hclrmix_oracle_trace.restype = I
        lib.hclrmix_oracle_trace.argtypes = common + [F] * 5 + [I64, P]
        lib.hclrmix_oracle_trace_floats.restype = I64
        lib.hclrmix_oracle_trace_floats.argtypes = [I64, I64, I64]
        lib.hclrmix_oracle_fp64.restype = I
        lib.hclrmix_oracle_fp64.argtypes = common + [D] * 5
        lib.hclrmix_oracle_round.restype = None
        lib.hclrmix_oracle_round.argtypes = [I, P, P, I64]
        lib.hclrmix_oracle_round_bits.restype = None
        lib.hclrmix_oracle_round_bits.argtypes = [I, ctypes.c_uint32, P, I64]
        lib.hclrmix_oracle_widen.restype = None
        lib.hclrmix_oracle_widen.argtypes = [I, P, P, I64]
        lib.hclrmix_oracle_sigmoid.restype = F
        lib.hclrmix_oracle_sigmoid.argtypes = [F]
        lib.hclrmix_oracle_inv_rms.restype = I
        lib.hclrmix_oracle_inv_rms.argtypes = [I, I64, I64, P, D, P]
        lib.hclrmix_oracle_inv_rms64.restype = I
        lib.hclrmix_oracle_inv_rms64.argtypes = [I, I64, I64, P, D, P]
        _lib = lib
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return t.data_ptr()


def _dims(streams, C, up_w):
    K = streams.shape[-1]
    rows = streams.numel() // K if K else 0
    return rows, K // C, up_w.shape[0]


def run(streams, norm_scale, down_w, up_w, inject_w, prev_out=None, prev_gate=None, *,
        num_branches: int, epsilon: float = 1e-5, reduction_scale: float = 1.0,
        silu_alpha: float = 1.0, gate_div: float = 1.0, gate_mul: float = 1.0,
        threads: int = 0, want_streams_out: bool = True, want_mag: bool = False):
    """(pre_output [rows,H], post_gate [rows,C], streams_out [rows,C*H]) in T, plus
    pre_mag [rows,H] (fp32, |rs| * sum_c |hn*g|) when want_mag."""
    dt = streams.dtype
    C = int(num_branches)
    rows, H, R = _dims(streams, C, up_w)
    pre = torch.empty(rows, H, dtype=dt)
    post = torch.empty(rows, C, dtype=dt)
    so = torch.empty(rows, C * H, dtype=dt) if want_streams_out else None
    mag = torch.empty(rows, H, dtype=torch.float32) if want_mag else None
    if threads <= 0:
        threads = default_threads()
    rc = _load().hclrmix_oracle_run_mag(
        DTYPE_CODE[dt], rows, C, H, R, _ptr(streams), _ptr(norm_scale), _ptr(down_w), _ptr(up_w),
        _ptr(inject_w), _ptr(prev_out), _ptr(prev_gate), _ptr(pre), _ptr(post), _ptr(so),
        epsilon, reduction_scale, silu_alpha, gate_div, gate_mul, int(threads), _ptr(mag))
    if rc != 0:
        raise ValueError(f"hclrmix_oracle_run failed with {rc}")
    if want_mag:
        return pre, post, so, mag
    return pre, post, so


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


TRACE_FIELDS = ("S", "hn", "down", "inject", "Z", "SG", "hidden", "up", "g", "pre", "post", "ss")


def trace(streams, norm_scale, down_w, up_w, inject_w, prev_out=None, prev_gate=None, *,
          row: int = 0, num_branches: int, epsilon: float = 1e-5, reduction_scale: float = 1.0,
          silu_alpha: float = 1.0, gate_div: float = 1.0, gate_mul: float = 1.0) -> dict:
    """Intermediates of one row, as fp32 tensors holding T values (ss is the raw fp32 sum)."""
    dt = streams.dtype
    C = int(num_branches)
    rows, H, R = _dims(streams, C, up_w)
    K = C * H
    lib = _load()
    buf = torch.empty(int(lib.hclrmix_oracle_trace_floats(C, H, R)), dtype=torch.float32)
    pre = torch.empty(rows, H, dtype=dt)
    post = torch.empty(rows, C, dtype=dt)
    rc = lib.hclrmix_oracle_trace(
        DTYPE_CODE[dt], rows, C, H, R, _ptr(streams), _ptr(norm_scale), _ptr(down_w), _ptr(up_w),
        _ptr(inject_w), _ptr(prev_out), _ptr(prev_gate), _ptr(pre), _ptr(post), None,
        epsilon, reduction_scale, silu_alpha, gate_div, gate_mul, int(row), _ptr(buf))
    if rc != 0:
        raise ValueError(f"hclrmix_oracle_trace failed with {rc}")
    sizes = (K, K, R, C, R, R, R, K, K, H, C, C)
    out, o = {}, 0
    for name, n in zip(TRACE_FIELDS, sizes):
        out[name] = buf[o:o + n].clone()
        o += n
    return out


def fp64(streams, norm_scale, down_w, up_w, inject_w, prev_out=None, prev_gate=None, *,
         num_branches: int, epsilon: float = 1e-5, reduction_scale: float = 1.0,
         silu_alpha: float = 1.0, gate_div: float = 1.0, gate_mul: float = 1.0):
    """The same algebra in float64 with no rounding to T."""
    dt = streams.dtype
    C = int(num_branches)
    rows, H, R = _dims(streams, C, up_w)
    pre = torch.empty(rows, H, dtype=torch.float64)
    post = torch.empty(rows, C, dtype=torch.float64)
    so = torch.empty(rows, C * H, dtype=torch.float64)
    rc = _load().hclrmix_oracle_fp64(
        DTYPE_CODE[dt], rows, C, H, R, _ptr(streams), _ptr(norm_scale), _ptr(down_w), _ptr(up_w),
        _ptr(inject_w), _ptr(prev_out), _ptr(prev_gate), _ptr(pre), _ptr(post), _ptr(so),
        epsilon, reduction_scale, silu_alpha, gate_div, gate_mul)
    if rc != 0:
        raise ValueError(f"hclrmix_oracle_fp64 failed with {rc}")
    return pre, post, so


def round_bits(dtype: torch.dtype, first: int, n: int) -> torch.Tensor:
    """Oracle's rounding of the fp32 bit patterns [first, first+n) to T (raw uint16 as int16)."""
    out = torch.empty(n, dtype=torch.int16)
    _load().hclrmix_oracle_round_bits(DTYPE_CODE[dtype], first, out.data_ptr(), n)
    return out


def round_values(dtype: torch.dtype, x: torch.Tensor) -> torch.Tensor:
    x = x.to(torch.float32).contiguous()
    out = torch.empty(x.numel(), dtype=torch.int16)
    _load().hclrmix_oracle_round(DTYPE_CODE[dtype], x.data_ptr(), out.data_ptr(), x.numel())
    return out.view(dtype).reshape(x.shape)


def widen_bits(dtype: torch.dtype, bits: torch.Tensor) -> torch.Tensor:
    bits = bits.contiguous()
    out = torch.empty(bits.numel(), dtype=torch.float32)
    _load().hclrmix_oracle_widen(DTYPE_CODE[dtype], bits.data_ptr(), out.data_ptr(), bits.numel())
    return out


def sigmoid(x: float) -> float:
    return float(_load().hclrmix_oracle_sigmoid(float(x)))


def inv_rms(x: torch.Tensor, eps: float, fp64: bool = False) -> torch.Tensor:
    """1 / sqrt(mean(x^2, last dim) + eps) per row of x [rows, dim] (T), taken in
    fp64 and rounded once to fp32 (fp64=True: the fp64 value itself)."""
    assert x.dim() == 2
    rows, dim = x.shape
    out = torch.empty(rows, dtype=torch.float64 if fp64 else torch.float32)
    fn = _load().hclrmix_oracle_inv_rms64 if fp64 else _load().hclrmix_oracle_inv_rms
    rc = fn(DTYPE_CODE[x.dtype], rows, dim, _ptr(x), float(eps), _ptr(out))
    if rc != 0:
        raise ValueError(f"inv_rms oracle failed with {rc}")
    return out
