"""Python binding of libhclrmix (the HyperConnectionLowRankMix block on MI355X).

Argument marshalling only: every step of the block runs in the HIP kernels
behind ``libhclrmix.so``. Functions carry the C-ABI names
(``include/hclrmix.h``); tensors are torch tensors on the GPU and the call is
enqueued on torch's current stream. There is no fallback: if the library is
missing, importing a function that needs it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhclrmix.so")

HCLRMIX_OK = 0
HCLRMIX_ERR_INVALID_ARGUMENT = 1
HCLRMIX_ERR_UNSUPPORTED = 2
HCLRMIX_ERR_WORKSPACE_TOO_SMALL = 3
HCLRMIX_ERR_DEVICE = 4

HCLRMIX_F32, HCLRMIX_F16, HCLRMIX_BF16 = 1, 10, 16
PATH_AUTO, PATH_DECODE, PATH_PREFILL, PATH_GENERIC = 0, 1, 2, 3
PATHS = {"auto": PATH_AUTO, "decode": PATH_DECODE, "prefill": PATH_PREFILL, "generic": PATH_GENERIC}
DECODE_MAX_ROWS = 16

EXPORTED = ("hclrmix_attrs_init", "hclrmix_infer_shapes", "hclrmix_select_path",
            "hclrmix_workspace_size", "hclrmix_hidden_offset", "hclrmix_run", "hclrmix_run_timed",
            "hclrmix_run_chained", "hclrmix_run_noalloc", "hclrmix_inv_rms", "hclrmix_status_string",
            "hclrmix_last_error", "hclrmix_version")
MAX_KERNELS = 7


class Attrs(ctypes.Structure):
    _fields_ = [("num_branches", ctypes.c_int64), ("epsilon", ctypes.c_float),
                ("reduction_scale", ctypes.c_float), ("silu_alpha", ctypes.c_float),
                ("gate_div", ctypes.c_float), ("gate_mul", ctypes.c_float)]


class Problem(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("width", ctypes.c_int64), ("rank", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("has_prologue", ctypes.c_int32),
                ("path", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class HclrmixError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


_lib = None


def library(path: Optional[str] = None):
    """Load libhclrmix.so (raises if it was not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build() or "
                           f"hyper_connection_rank_amd/build.py")
    # torch first: its HIP runtime carries the same soname, so the library binds
    # to that one and torch's streams and events are valid handles for it.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    P, I32 = ctypes.c_void_p, ctypes.c_int
    lib.hclrmix_attrs_init.restype = None
    lib.hclrmix_attrs_init.argtypes = [ctypes.POINTER(Attrs)]
    pi64 = ctypes.POINTER(ctypes.c_int64)
    lib.hclrmix_infer_shapes.restype = I32
    lib.hclrmix_infer_shapes.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Attrs), pi64, pi64, pi64, pi64]
    lib.hclrmix_select_path.restype = I32
    lib.hclrmix_select_path.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Attrs),
                                        ctypes.POINTER(ctypes.c_int32)]
    lib.hclrmix_workspace_size.restype = I32
    lib.hclrmix_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Attrs),
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.hclrmix_hidden_offset.restype = I32
    lib.hclrmix_hidden_offset.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Attrs),
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.hclrmix_run.restype = I32
    lib.hclrmix_run.argtypes = [P] * 11 + [ctypes.c_size_t, ctypes.POINTER(Problem), ctypes.POINTER(Attrs), P]
    lib.hclrmix_run_timed.restype = I32
    lib.hclrmix_run_timed.argtypes = ([P] * 11 + [ctypes.c_size_t, ctypes.POINTER(Problem), ctypes.POINTER(Attrs), P,
                                      ctypes.POINTER(ctypes.c_void_p), I32, ctypes.POINTER(I32)])
    lib.hclrmix_run_chained.restype = I32
    lib.hclrmix_run_chained.argtypes = ([P] * 11 + [ctypes.c_size_t, ctypes.POINTER(Problem), ctypes.POINTER(Attrs),
                                        P, P, P, ctypes.POINTER(ctypes.c_void_p), I32, ctypes.POINTER(I32)])
    lib.hclrmix_run_noalloc.restype = I32
    lib.hclrmix_run_noalloc.argtypes = [P] * 10 + [ctypes.POINTER(Problem), ctypes.POINTER(Attrs), P]
    lib.hclrmix_inv_rms.restype = I32
    lib.hclrmix_inv_rms.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, P]
    lib.hclrmix_status_string.restype = ctypes.c_char_p
    lib.hclrmix_status_string.argtypes = [I32]
    lib.hclrmix_last_error.restype = ctypes.c_char_p
    lib.hclrmix_last_error.argtypes = []
    lib.hclrmix_version.restype = ctypes.c_char_p
    lib.hclrmix_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return library().hclrmix_status_string(int(status)).decode()
    except Exception:
        return f"status {status}"


def _check(status: int):
    if status != HCLRMIX_OK:
        raise HclrmixError(status, library().hclrmix_last_error().decode())


def dtype_code(torch_dtype) -> int:
    import torch
    return {torch.float32: HCLRMIX_F32, torch.float16: HCLRMIX_F16, torch.bfloat16: HCLRMIX_BF16}[torch_dtype]


def make_attrs(num_branches: int, epsilon: float = 1e-5, reduction_scale: float = 1.0,
               silu_alpha: float = 1.0, gate_div: float = 1.0, gate_mul: float = 1.0) -> Attrs:
    a = Attrs()
    library().hclrmix_attrs_init(ctypes.byref(a))
    a.num_branches = int(num_branches)
    a.epsilon, a.reduction_scale, a.silu_alpha = float(epsilon), float(reduction_scale), float(silu_alpha)
    a.gate_div, a.gate_mul = float(gate_div), float(gate_mul)
    return a


def make_problem(rows: int, width: int, rank: int, dtype: int, has_prologue: bool, path="auto") -> Problem:
    p = Problem()
    p.rows, p.width, p.rank, p.dtype = int(rows), int(width), int(rank), int(dtype)
    p.has_prologue = 1 if has_prologue else 0
    p.path = PATHS[path] if isinstance(path, str) else int(path)
    p.reserved = 0
    return p


def hclrmix_attrs_init() -> Attrs:
    a = Attrs()
    library().hclrmix_attrs_init(ctypes.byref(a))
    return a


def hclrmix_infer_shapes(problem: Problem, attrs: Attrs) -> Tuple[int, int, int, int]:
    h, pc, gc, sc = (ctypes.c_int64() for _ in range(4))
    _check(library().hclrmix_infer_shapes(ctypes.byref(problem), ctypes.byref(attrs), ctypes.byref(h),
                                          ctypes.byref(pc), ctypes.byref(gc), ctypes.byref(sc)))
    return h.value, pc.value, gc.value, sc.value


def hclrmix_select_path(problem: Problem, attrs: Attrs) -> int:
    p = ctypes.c_int32()
    _check(library().hclrmix_select_path(ctypes.byref(problem), ctypes.byref(attrs), ctypes.byref(p)))
    return p.value


def hclrmix_workspace_size(problem: Problem, attrs: Attrs) -> int:
    n = ctypes.c_size_t()
    _check(library().hclrmix_workspace_size(ctypes.byref(problem), ctypes.byref(attrs), ctypes.byref(n)))
    return n.value


def hclrmix_hidden_offset(problem: Problem, attrs: Attrs) -> int:
    """Byte offset of hidden [rows, R] (T) inside the workspace after a call."""
    n = ctypes.c_size_t()
    _check(library().hclrmix_hidden_offset(ctypes.byref(problem), ctypes.byref(attrs), ctypes.byref(n)))
    return n.value


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def hclrmix_run(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output,
                prev_post_gate, pre_output, post_gate, streams_out, workspace, problem: Problem,
                attrs: Attrs, stream=None) -> None:
    """Enqueue one block on ``stream`` (default: torch's current stream)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(streams.device).cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().hclrmix_run(
        _ptr(streams), _ptr(norm_scale), _ptr(down_weight), _ptr(up_weight), _ptr(inject_weight),
        _ptr(prev_block_output), _ptr(prev_post_gate), _ptr(pre_output), _ptr(post_gate),
        _ptr(streams_out), _ptr(workspace), ws_bytes, ctypes.byref(problem), ctypes.byref(attrs),
        ctypes.c_void_p(int(stream))))


def hclrmix_run_timed(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output,
                      prev_post_gate, pre_output, post_gate, streams_out, workspace, problem: Problem,
                      attrs: Attrs, events, stream=None) -> int:
    """hclrmix_run whose i-th kernel is dispatched with the raw hipEvent_t
    handles events[2i] / events[2i+1] (at least 2 * MAX_KERNELS of them) as its
    start and stop events; returns the number of kernels."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(streams.device).cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * len(events))(*[int(e) for e in events])
    k = ctypes.c_int(0)
    _check(library().hclrmix_run_timed(
        _ptr(streams), _ptr(norm_scale), _ptr(down_weight), _ptr(up_weight), _ptr(inject_weight),
        _ptr(prev_block_output), _ptr(prev_post_gate), _ptr(pre_output), _ptr(post_gate),
        _ptr(streams_out), _ptr(workspace), ws_bytes, ctypes.byref(problem), ctypes.byref(attrs),
        ctypes.c_void_p(int(stream)), arr, len(events), ctypes.byref(k)))
    return k.value


def hclrmix_run_chained(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output,
                        prev_post_gate, pre_output, post_gate, streams_out, workspace, problem: Problem,
                        attrs: Attrs, next_down_weight=None, next_inject_weight=None, events=None,
                        stream=None) -> int:
    """hclrmix_run for one block of a chain that also brings the next block's
    down_weight / inject_weight into cache (None: not that one); with events
    (raw hipEvent_t handles, at least 2 * MAX_KERNELS) it is timed like
    hclrmix_run_timed. Returns the number of kernels (0 when untimed)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(streams.device).cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    k = ctypes.c_int(0)
    if events is None:
        arr, n, kp = None, 0, None
    else:
        arr, n, kp = (ctypes.c_void_p * len(events))(*[int(e) for e in events]), len(events), ctypes.byref(k)
    _check(library().hclrmix_run_chained(
        _ptr(streams), _ptr(norm_scale), _ptr(down_weight), _ptr(up_weight), _ptr(inject_weight),
        _ptr(prev_block_output), _ptr(prev_post_gate), _ptr(pre_output), _ptr(post_gate),
        _ptr(streams_out), _ptr(workspace), ws_bytes, ctypes.byref(problem), ctypes.byref(attrs),
        _ptr(next_down_weight), _ptr(next_inject_weight), ctypes.c_void_p(int(stream)), arr, n, kp))
    return k.value


NOALLOC_SCRATCH_BYTES = 16 << 20


def hclrmix_run_noalloc(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output,
                        prev_post_gate, pre_output, post_gate, streams_out, problem: Problem, attrs: Attrs,
                        stream=None) -> None:
    """hclrmix_run with the library's static scratch instead of a workspace
    (no allocation; calls on one GPU must not overlap)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(streams.device).cuda_stream
    _check(library().hclrmix_run_noalloc(
        _ptr(streams), _ptr(norm_scale), _ptr(down_weight), _ptr(up_weight), _ptr(inject_weight),
        _ptr(prev_block_output), _ptr(prev_post_gate), _ptr(pre_output), _ptr(post_gate),
        _ptr(streams_out), ctypes.byref(problem), ctypes.byref(attrs), ctypes.c_void_p(int(stream))))


def hclrmix_inv_rms(x, eps: float, out=None, stream=None):
    """1 / sqrt(mean(x^2, last dim) + eps) per row of x, one fp32 value each.
    x: a GPU tensor (fp32, fp16 or bf16) of shape [..., dim], contiguous; the
    leading dimensions are flattened into rows. Returns out [rows] (fp32)."""
    import torch
    assert x.is_contiguous()
    dim = x.shape[-1] if x.dim() else 1
    rows = x.numel() // dim if dim else 0
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _check(library().hclrmix_inv_rms(_ptr(x), _ptr(out), rows, dim, dtype_code(x.dtype), float(eps),
                                     ctypes.c_void_p(int(stream))))
    return out


def hclrmix_status_string(status: int) -> str:
    return status_string(status)


def hclrmix_last_error() -> str:
    return library().hclrmix_last_error().decode()


def hclrmix_version() -> str:
    return library().hclrmix_version().decode()


def new_workspace(problem: Problem, attrs: Attrs, device):
    """A zero-filled device workspace for ``problem`` (zero it once; calls keep it valid)."""
    import torch
    return torch.zeros(max(hclrmix_workspace_size(problem, attrs), 1), dtype=torch.uint8, device=device)


def block(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output=None,
          prev_post_gate=None, *, num_branches: int, epsilon: float = 1e-5,
          reduction_scale: float = 1.0, silu_alpha: float = 1.0, gate_div: float = 1.0,
          gate_mul: float = 1.0, want_streams_out: bool = True, path="auto", out=None, workspace=None):
    """One block with torch-allocated outputs: returns (pre_output, post_gate, streams_out).

    ``out`` may supply (pre_output, post_gate, streams_out) buffers and
    ``workspace`` a zero-filled (before first use) uint8 device buffer of at
    least hclrmix_workspace_size bytes, e.g. from new_workspace().
    """
    import torch
    K = streams.shape[-1]
    lead = streams.shape[:-1]
    rows = streams.numel() // K if K else 0
    R = up_weight.shape[0]
    attrs = make_attrs(num_branches, epsilon, reduction_scale, silu_alpha, gate_div, gate_mul)
    prob = make_problem(rows, K, R, dtype_code(streams.dtype), prev_block_output is not None, path)
    H, _, C, _ = hclrmix_infer_shapes(prob, attrs)
    if out is None:
        pre = torch.empty(*lead, H, dtype=streams.dtype, device=streams.device)
        post = torch.empty(*lead, C, dtype=streams.dtype, device=streams.device)
        so = torch.empty_like(streams) if want_streams_out else None
    else:
        pre, post, so = out
    if workspace is None:
        workspace = new_workspace(prob, attrs, streams.device)
    hclrmix_run(streams, norm_scale, down_weight, up_weight, inject_weight, prev_block_output,
                prev_post_gate, pre, post, so, workspace, prob, attrs)
    return pre, post, so
