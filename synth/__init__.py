"""Seeded synthetic inputs for the HyperConnectionLowRankMix block.

This module only produces input tensors; it contains none of the block's
arithmetic. Both sides of every parity check (the HIP library and the CPU
oracle) receive the bytes it returns, so they never disagree about inputs.

Recipe (every tensor): float32 values drawn by ``hclrmix_synth.c``
(counter-based SplitMix64 feeding Box-Muller normals or uniforms), then
rounded to the element type T with round-to-nearest-even by torch's dtype
conversion. Per-tensor seed::

    seed = 20261202 + 1000003 * workload + 10007 * block + tensor_id

with tensor ids streams=0, norm_scale=1, down=2, up=3, inject=4,
prev_out=5, prev_gate=6.

Distributions (the shapes and attribute values of the Qwen3.8-Flash-Next
block in onnxruntime PR #33384, "Description" and "Schema summary"; the
pages print no input values, so values are synthetic):

* streams ~ N(0, streams_std^2), prev_out ~ N(0, 1), prev_gate ~ U(0, 2)
* norm_scale = 1 + U(-0.1, 0.1) over [C*H]
* down, inject ~ N(0, 1/(C*H)), up ~ N(0, 1/R)  (fan-in scaled)
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhclrmix_synth.so")

TENSOR_IDS = {
    "streams": 0,
    "norm_scale": 1,
    "down_weight": 2,
    "up_weight": 3,
    "inject_weight": 4,
    "prev_block_output": 5,
    "prev_post_gate": 6,
}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: run __graft_entry__.build() (or synth/build.py) first")
        lib = ctypes.CDLL(LIB_PATH)
        for name in ("hcs_fill_normal", "hcs_fill_uniform"):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                           ctypes.c_double, ctypes.c_double, ctypes.c_int]
        lib.hcs_splitmix64.restype = ctypes.c_uint64
        lib.hcs_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        _lib = lib
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal(n: int, seed: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(int(n), dtype=np.float32)
    _load().hcs_fill_normal(out.ctypes.data, int(n), int(seed) & (2**64 - 1),
                            float(mean), float(std), _threads())
    return out


def uniform(n: int, seed: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(int(n), dtype=np.float32)
    _load().hcs_fill_uniform(out.ctypes.data, int(n), int(seed) & (2**64 - 1),
                             float(lo), float(hi), _threads())
    return out


def splitmix64(seed: int, counter: int) -> int:
    return int(_load().hcs_splitmix64(int(seed) & (2**64 - 1), int(counter) & (2**64 - 1)))


def seed_for(workload: int, block: int, tensor: str) -> int:
    return 20261202 + 1000003 * int(workload) + 10007 * int(block) + TENSOR_IDS[tensor]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One block shape with its attributes and input distributions."""
    wid: int                 # workload id used in the seed
    name: str
    rows: int
    C: int
    H: int
    R: int
    dtype: str               # "f32" | "f16" | "bf16"
    has_prologue: bool
    epsilon: float
    reduction_scale: float
    silu_alpha: float
    gate_div: float
    gate_mul: float
    streams_std: float = 1.0
    blocks: int = 1          # chained blocks (decode chain)

    @property
    def K(self) -> int:
        return self.C * self.H

    def attrs(self) -> dict:
        return dict(num_branches=self.C, epsilon=self.epsilon,
                    reduction_scale=self.reduction_scale, silu_alpha=self.silu_alpha,
                    gate_div=self.gate_div, gate_mul=self.gate_mul)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_QWEN_ATTRS = dict(epsilon=1e-6, reduction_scale=0.25, silu_alpha=0.25, gate_div=4.0, gate_mul=2.0)

WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload(0, "tiny fp32 block rows=2 C=4 H=64 R=16 prologue", 2, 4, 64, 16, "f32", True, **_QWEN_ATTRS),
    "decode_bf16": Workload(1, "decode bf16 rows=1 C=4 H=2560 R=320 prologue", 1, 4, 2560, 320, "bf16", True, **_QWEN_ATTRS),
    "decode_chain_bf16": Workload(2, "decode chain bf16 rows=8 C=4 H=2560 R=320 x96 blocks", 8, 4, 2560, 320, "bf16", True,
                                  blocks=96, **_QWEN_ATTRS),
    "prefill_bf16": Workload(3, "prefill bf16 rows=8192 C=4 H=2560 R=320 prologue", 8192, 4, 2560, 320, "bf16", True, **_QWEN_ATTRS),
    "wide_f16": Workload(4, "wide fp16 rows=64 C=8 H=4096 R=512 no prologue", 64, 8, 4096, 512, "f16", False,
                         epsilon=1e-5, reduction_scale=1.0, silu_alpha=1.0, gate_div=1.0, gate_mul=1.0,
                         streams_std=4.0),
}


def block_inputs_f32(w: Workload, block: int = 0, rows: Optional[int] = None,
                     with_weights: bool = True, with_acts: bool = True) -> Dict[str, np.ndarray]:
    """float32 values of every input of block ``block`` (before rounding to T)."""
    M = w.rows if rows is None else int(rows)
    K, H, C, R = w.K, w.H, w.C, w.R
    s = lambda name: seed_for(w.wid, block, name)  # noqa: E731
    out: Dict[str, np.ndarray] = {}
    if with_acts:
        out["streams"] = normal(M * K, s("streams"), 0.0, w.streams_std).reshape(M, K)
        if w.has_prologue:
            out["prev_block_output"] = normal(M * H, s("prev_block_output"), 0.0, 1.0).reshape(M, H)
            out["prev_post_gate"] = uniform(M * C, s("prev_post_gate"), 0.0, 2.0).reshape(M, C)
    if with_weights:
        out["norm_scale"] = uniform(K, s("norm_scale"), 0.9, 1.1)
        out["down_weight"] = normal(K * R, s("down_weight"), 0.0, 1.0 / np.sqrt(K)).reshape(K, R)
        out["up_weight"] = normal(R * K, s("up_weight"), 0.0, 1.0 / np.sqrt(R)).reshape(R, K)
        out["inject_weight"] = normal(K * C, s("inject_weight"), 0.0, 1.0 / np.sqrt(K)).reshape(K, C)
    return out


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_t(a: np.ndarray, dtype: str):
    """Round float32 values to T (round-to-nearest-even) as a CPU torch tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(dtype)).contiguous()


def block_inputs(w: Workload, block: int = 0, rows: Optional[int] = None,
                 with_weights: bool = True, with_acts: bool = True):
    """Inputs of block ``block`` as CPU torch tensors of element type T."""
    return {k: to_t(v, w.dtype) for k, v in
            block_inputs_f32(w, block, rows, with_weights, with_acts).items()}
