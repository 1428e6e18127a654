"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, applies the shape rule, sizes workspaces per path, selects
paths, and rejects every invalid call on the host before any GPU work (fake,
never-dereferenced device pointers are enough for that)."""
from __future__ import annotations

import ctypes
import json
import os
import re

import pytest

import hyper_connection_rank_amd as hc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_declared_symbol_is_exported():
    header = open(os.path.join(ROOT, "include", "hclrmix.h")).read()
    body = header[header.index('extern "C" {'):]
    names = set(re.findall(r"\b(hclrmix_[a-z_0-9]+)\s*\(", body))
    assert names == set(hc.EXPORTED)
    lib = ctypes.CDLL(hc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert re.match(r"^\d+\.\d+\.\d+$", hc.hclrmix_version())


def test_measurement_library_exports_its_entry_points():
    # libhcpeaks (bench.py's achievable-peak kernels) is built beside libhclrmix
    # and exports no hclrmix_ symbol.
    from hyper_connection_rank_amd import build as B
    lib = ctypes.CDLL(B.PEAKS_LIB)
    for n in ("hcpeaks_read", "hcpeaks_copy", "hcpeaks_mfma_bf16", "hcpeaks_empty", "hcpeaks_stream",
              "hcpeaks_overlap"):
        assert hasattr(lib, n), n
    assert not hasattr(lib, "hclrmix_run")


def test_attrs_defaults_follow_schema():
    a = hc.hclrmix_attrs_init()
    assert a.num_branches == 0
    assert abs(a.epsilon - 1e-5) < 1e-12
    assert (a.reduction_scale, a.silu_alpha, a.gate_div, a.gate_mul) == (1.0, 1.0, 1.0, 1.0)


def test_shape_rule_golden_review_example():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "shape_inference_review.json")))
    attrs = hc.make_attrs(g["num_branches"])
    for rows in (0, 1, 7):
        prob = hc.make_problem(rows, g["streams"][1], g["down_weight"][1], hc.HCLRMIX_F32, False)
        H, pre, post, so = hc.hclrmix_infer_shapes(prob, attrs)
        assert (pre, post, so) == (g["expect"]["pre_output_last"], g["expect"]["post_gate_last"],
                                   g["expect"]["streams_out_last"])
        assert H == g["streams"][1] // g["num_branches"]


@pytest.mark.parametrize("width,C,rank,status", [
    (16, 0, 8, hc.HCLRMIX_ERR_INVALID_ARGUMENT),
    (15, 2, 8, hc.HCLRMIX_ERR_INVALID_ARGUMENT),
    (16, 2, 0, hc.HCLRMIX_ERR_INVALID_ARGUMENT),
    (0, 2, 8, hc.HCLRMIX_ERR_INVALID_ARGUMENT),
])
def test_shape_rule_errors(width, C, rank, status):
    with pytest.raises(hc.HclrmixError) as e:
        hc.hclrmix_infer_shapes(hc.make_problem(3, width, rank, hc.HCLRMIX_BF16, False), hc.make_attrs(C))
    assert e.value.status == status


@pytest.mark.parametrize("dtype,C,H,R,rows,expect", [
    (hc.HCLRMIX_BF16, 4, 2560, 320, 1, hc.PATH_DECODE),
    (hc.HCLRMIX_BF16, 4, 2560, 320, 16, hc.PATH_DECODE),
    (hc.HCLRMIX_BF16, 4, 2560, 320, 17, hc.PATH_PREFILL),
    (hc.HCLRMIX_F16, 8, 4096, 512, 64, hc.PATH_PREFILL),
    (hc.HCLRMIX_F32, 4, 64, 16, 2, hc.PATH_GENERIC),
    (hc.HCLRMIX_BF16, 4, 48, 32, 1, hc.PATH_DECODE),      # H % 32 != 0: zero-padded
    (hc.HCLRMIX_BF16, 4, 64, 24, 1, hc.PATH_DECODE),      # R % 32 != 0: zero-padded
    (hc.HCLRMIX_F16, 3, 33, 8, 17, hc.PATH_PREFILL),      # both, many rows
    (hc.HCLRMIX_F32, 4, 48, 24, 1, hc.PATH_GENERIC),      # fp32 is never padded
    (hc.HCLRMIX_BF16, 1, 8190, 64, 1, hc.PATH_DECODE),    # padded to 8192 features
    (hc.HCLRMIX_BF16, 1, 8193, 64, 1, hc.PATH_PREFILL),   # padded beyond the decode kernels' width
    (hc.HCLRMIX_BF16, 16, 64, 32, 1, hc.PATH_GENERIC),    # C > 8
    (hc.HCLRMIX_BF16, 4, 64, 544, 1, hc.PATH_GENERIC),    # R > 512
    (hc.HCLRMIX_BF16, 1, 8192, 64, 1, hc.PATH_DECODE),    # widest branch the decode kernels take
    (hc.HCLRMIX_BF16, 1, 8224, 64, 1, hc.PATH_PREFILL),   # wider branches: few rows go to prefill
])
def test_auto_path_selection(dtype, C, H, R, rows, expect):
    assert hc.hclrmix_select_path(hc.make_problem(rows, C * H, R, dtype, True), hc.make_attrs(C)) == expect


def test_forced_matrix_core_path_outside_envelope_is_unsupported():
    with pytest.raises(hc.HclrmixError) as e:
        hc.hclrmix_select_path(hc.make_problem(4, 4 * 64, 16, hc.HCLRMIX_F32, True, "decode"), hc.make_attrs(4))
    assert e.value.status == hc.HCLRMIX_ERR_UNSUPPORTED
    with pytest.raises(hc.HclrmixError) as e:
        hc.hclrmix_select_path(hc.make_problem(17, 4 * 64, 32, hc.HCLRMIX_BF16, True, "decode"), hc.make_attrs(4))
    assert e.value.status == hc.HCLRMIX_ERR_UNSUPPORTED
    assert hc.hclrmix_select_path(hc.make_problem(17, 4 * 64, 32, hc.HCLRMIX_BF16, True, "prefill"),
                                  hc.make_attrs(4)) == hc.PATH_PREFILL
    with pytest.raises(hc.HclrmixError) as e:
        hc.hclrmix_select_path(hc.make_problem(1, 8224, 64, hc.HCLRMIX_BF16, True, "decode"), hc.make_attrs(1))
    assert e.value.status == hc.HCLRMIX_ERR_UNSUPPORTED
    # zero-padded shapes: forced decode up to 8192 padded features, forced
    # prefill beyond; never more than 8 branches or rank 512
    assert hc.hclrmix_select_path(hc.make_problem(3, 4 * 48, 24, hc.HCLRMIX_F16, True, "decode"),
                                  hc.make_attrs(4)) == hc.PATH_DECODE
    assert hc.hclrmix_select_path(hc.make_problem(3, 8193, 24, hc.HCLRMIX_BF16, True, "prefill"),
                                  hc.make_attrs(1)) == hc.PATH_PREFILL
    for rows, width, rank, C in ((1, 8193, 64, 1), (1, 9 * 40, 24, 9), (1, 4 * 40, 513, 4)):
        with pytest.raises(hc.HclrmixError) as e:
            hc.hclrmix_select_path(hc.make_problem(rows, width, rank, hc.HCLRMIX_BF16, True, "decode"),
                                   hc.make_attrs(C))
        assert e.value.status == hc.HCLRMIX_ERR_UNSUPPORTED


def test_workspace_sized_per_path():
    attrs = hc.make_attrs(4)
    bf16 = hc.HCLRMIX_BF16

    def size(rows, path, dtype=bf16):
        return hc.hclrmix_workspace_size(hc.make_problem(rows, 10240, 320, dtype, True, path), attrs)

    part = lambda n, rows: n * rows * 336 * 4  # noqa: E731  fp32 partials, R + C padded to 336
    wut_tab = 10240 * 320 * 2 + 6144 * 2       # up_weight transposed and the sigmoid table
    # decode: one partial per slice (40 slices of 256) and hn
    assert size(8, "decode") >= part(40, 8) + 8 * 10240 * 2
    # prefill at 8 rows: one slice per down workgroup (40 partials), the plain up kernel
    assert part(40, 8) <= size(8, "prefill") < part(40, 8) + wut_tab
    # prefill at 600 rows: still slices, and the bf16 up kernel's transposed copy and table
    assert size(600, "prefill") >= part(40, 600) + wut_tab
    # prefill at 2100 rows: one partial per branch
    assert part(4, 2100) + wut_tab <= size(2100, "prefill") < part(40, 2100)
    # generic: rinv, hidden and one partial per part of K (16 parts of 640)
    assert size(8, "generic") >= 8 * 4 * 4 + 8 * 320 * 2 + 16 * 8 * 324 * 4
    # fp16 prefill takes the other up kernel: no transposed copy
    assert size(2100, "prefill", hc.HCLRMIX_F16) < part(4, 2100) + 10240 * 320 * 2
    assert hc.hclrmix_workspace_size(hc.make_problem(0, 10240, 320, hc.HCLRMIX_BF16, True), attrs) == 0


def test_workspace_of_a_zero_padded_problem():
    """H = 2056 and R = 328 run as 2080 and 352: the workspace holds the padded
    problem's own workspace, the padded copies of streams, the prologue
    inputs, norm_scale, the three weights and the outputs, then hidden
    [rows, R], whose offset the caller reads."""
    attrs = hc.make_attrs(4)

    def problem(rows, H, R, path, pro=True):
        return hc.make_problem(rows, 4 * H, R, hc.HCLRMIX_BF16, pro, path)

    for path, rows in (("decode", 5), ("prefill", 40), ("prefill", 700)):
        K32 = 4 * 2080
        copies = 2 * (rows * K32 + rows * 2080 + rows * 4 + K32 + 2 * K32 * 352 + K32 * 4  # inputs
                      + rows * 2080 + rows * 4 + rows * K32)                               # outputs
        inner = hc.hclrmix_workspace_size(problem(rows, 2080, 352, path), attrs)
        size = hc.hclrmix_workspace_size(problem(rows, 2056, 328, path), attrs)
        assert size >= inner + copies + rows * 328 * 2, path
        assert size < inner + copies + rows * 328 * 2 + 12 * 256, path
        off = hc.hclrmix_hidden_offset(problem(rows, 2056, 328, path), attrs)
        assert off >= inner + copies and off + rows * 328 * 2 <= size, path
        # without a prologue there are no prologue copies
        assert hc.hclrmix_workspace_size(problem(rows, 2056, 328, path, False), attrs) < size
    # rows = 0 needs none
    assert hc.hclrmix_workspace_size(problem(0, 2056, 328, "auto"), attrs) == 0


# ----------------------------------------------------------------------------- hclrmix_run validation

BASE = 1 << 40  # fake device addresses, 16-byte aligned, far apart; never dereferenced


class Call:
    def __init__(self, rows=2, C=4, H=64, R=32, dtype=hc.HCLRMIX_BF16, prologue=True, path="auto"):
        self.p = {n: BASE + i * (1 << 30) for i, n in enumerate(
            ["streams", "ns", "wd", "wu", "wi", "po", "pg", "pre", "post", "so", "ws"])}
        if not prologue:
            self.p["po"] = self.p["pg"] = None
        self.prob = hc.make_problem(rows, C * H, R, dtype, prologue, path)
        self.attrs = hc.make_attrs(C, 1e-6, 0.25, 0.25, 4.0, 2.0)
        self.ws_bytes = 1 << 30

    def run(self):
        p = self.p
        v = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
        return hc.library().hclrmix_run(
            v(p["streams"]), v(p["ns"]), v(p["wd"]), v(p["wu"]), v(p["wi"]), v(p["po"]), v(p["pg"]),
            v(p["pre"]), v(p["post"]), v(p["so"]), v(p["ws"]), self.ws_bytes, ctypes.byref(self.prob),
            ctypes.byref(self.attrs), None)


def _expect(call, status, fragment=""):
    assert call.run() == status
    if fragment:
        assert fragment in hc.hclrmix_last_error()


def test_zero_rows_returns_ok_without_launching():
    c = Call(rows=0)
    for k in c.p:
        c.p[k] = None
    c.prob.has_prologue = 0
    c.ws_bytes = 0
    _expect(c, hc.HCLRMIX_OK)


@pytest.mark.parametrize("missing", ["streams", "ns", "wd", "wu", "wi", "pre", "post"])
def test_required_pointers(missing):
    c = Call()
    c.p[missing] = None
    _expect(c, hc.HCLRMIX_ERR_INVALID_ARGUMENT, "required")


@pytest.mark.parametrize("drop", ["po", "pg"])
def test_prologue_inputs_come_as_a_pair(drop):
    c = Call()
    c.p[drop] = None
    _expect(c, hc.HCLRMIX_ERR_INVALID_ARGUMENT, "together")


def test_prologue_flag_must_match_pointers():
    c = Call(prologue=True)
    c.prob.has_prologue = 0
    _expect(c, hc.HCLRMIX_ERR_INVALID_ARGUMENT, "has_prologue")


@pytest.mark.parametrize("field,value", [("gate_div", 0.0), ("epsilon", float("nan")),
                                         ("gate_mul", float("inf")), ("reduction_scale", float("-inf")),
                                         ("silu_alpha", float("nan"))])
def test_bad_attributes(field, value):
    c = Call()
    setattr(c.attrs, field, value)
    _expect(c, hc.HCLRMIX_ERR_INVALID_ARGUMENT)


def test_reserved_and_unknown_path_and_dtype():
    c = Call()
    c.prob.reserved = 1
    _expect(c, hc.HCLRMIX_ERR_INVALID_ARGUMENT, "reserved")
    c = Call()
    c.prob.path = 9
    _expect(c, hc.HCLRMIX_ERR_INVALID_ARGUMENT, "path")
    c = Call()
    c.prob.dtype = 11
    _expect(c, hc.HCLRMIX_ERR_UNSUPPORTED, "dtype")


@pytest.mark.parametrize("out", ["pre", "post", "so", "ws"])
@pytest.mark.parametrize("other", ["streams", "wd", "po", "pre", "so"])
def test_outputs_must_not_overlap(out, other):
    if out == other:
        return
    c = Call()
    c.p[out] = c.p[other] + 16
    _expect(c, hc.HCLRMIX_ERR_INVALID_ARGUMENT, "overlaps")


def test_workspace_too_small():
    c = Call()
    need = hc.hclrmix_workspace_size(c.prob, c.attrs)
    c.ws_bytes = need - 1
    _expect(c, hc.HCLRMIX_ERR_WORKSPACE_TOO_SMALL, str(need))
    c = Call()
    c.p["ws"] = None
    _expect(c, hc.HCLRMIX_ERR_WORKSPACE_TOO_SMALL)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_matrix_core_paths_need_16_byte_alignment(path):
    c = Call(path=path)
    c.p["streams"] += 2
    _expect(c, hc.HCLRMIX_ERR_UNSUPPORTED, "aligned")


def test_generic_path_needs_element_alignment_only():
    c = Call(dtype=hc.HCLRMIX_F32, path="generic")
    c.p["wd"] += 2
    _expect(c, hc.HCLRMIX_ERR_UNSUPPORTED, "element-aligned")


def test_status_strings():
    assert hc.hclrmix_status_string(hc.HCLRMIX_OK) == "ok"
    assert hc.hclrmix_status_string(hc.HCLRMIX_ERR_WORKSPACE_TOO_SMALL) == "workspace too small"


def _chained(c, next_wd, next_wi, events=None, n_events=0, kernels=None):
    p = c.p
    v = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return hc.library().hclrmix_run_chained(
        v(p["streams"]), v(p["ns"]), v(p["wd"]), v(p["wu"]), v(p["wi"]), v(p["po"]), v(p["pg"]),
        v(p["pre"]), v(p["post"]), v(p["so"]), v(p["ws"]), c.ws_bytes, ctypes.byref(c.prob),
        ctypes.byref(c.attrs), v(next_wd), v(next_wi), None, events, n_events, kernels)


def test_chained_call_validates_like_run_and_checks_next_weights():
    """hclrmix_run_chained applies hclrmix_run's checks, needs 16-byte aligned
    next-block weights on the decode path, and with events asks for enough of
    them and a kernels pointer (all refused before any launch)."""
    c = Call(path="decode")
    c.p["wd"] = None
    assert _chained(c, BASE, BASE) == hc.HCLRMIX_ERR_INVALID_ARGUMENT
    c = Call(path="decode")
    assert _chained(c, BASE + 8, None) == hc.HCLRMIX_ERR_UNSUPPORTED
    assert "next-block" in hc.hclrmix_last_error()
    assert _chained(c, None, BASE + 4) == hc.HCLRMIX_ERR_UNSUPPORTED
    ev = (ctypes.c_void_p * 2)()
    k = ctypes.c_int(0)
    assert _chained(c, None, None, ev, 2, ctypes.byref(k)) == hc.HCLRMIX_ERR_INVALID_ARGUMENT
    ev = (ctypes.c_void_p * (2 * hc.MAX_KERNELS))()
    assert _chained(c, None, None, ev, 2 * hc.MAX_KERNELS, None) == hc.HCLRMIX_ERR_INVALID_ARGUMENT


def _inv_rms(x, out, rows, dim, dtype=hc.HCLRMIX_BF16, eps=1e-6):
    v = lambda a: ctypes.c_void_p(a) if a is not None else None  # noqa: E731
    return hc.library().hclrmix_inv_rms(v(x), v(out), rows, dim, dtype, eps, None)


def test_inv_rms_validation():
    """hclrmix_inv_rms refuses bad arguments before any launch."""
    E, U, OK = hc.HCLRMIX_ERR_INVALID_ARGUMENT, hc.HCLRMIX_ERR_UNSUPPORTED, hc.HCLRMIX_OK
    x, o = BASE, BASE + (1 << 32)
    assert _inv_rms(None, None, 0, 16) == OK  # no rows: nothing to do
    assert _inv_rms(x, o, -1, 16) == E
    assert _inv_rms(x, o, 4, 0) == E
    assert _inv_rms(None, o, 4, 16) == E
    assert _inv_rms(x, None, 4, 16) == E
    assert _inv_rms(x, o, 4, 16, eps=float("nan")) == E
    assert _inv_rms(x, o, 4, 16, dtype=11) == U
    assert _inv_rms(x + 1, o, 4, 16) == U
    assert _inv_rms(x, o + 2, 4, 16) == U
    assert _inv_rms(x, x + 8, 4, 16) == E and "overlaps" in hc.hclrmix_last_error()


def test_noalloc_refuses_problems_beyond_its_scratch_on_the_host():
    # rows=8192 prefill needs ~53 MiB of scratch, more than the static array:
    # refused before any device call (fake, never-dereferenced pointers).
    attrs = hc.make_attrs(4)
    prob = hc.make_problem(8192, 10240, 320, hc.HCLRMIX_BF16, False)
    assert hc.hclrmix_workspace_size(prob, attrs) > hc.NOALLOC_SCRATCH_BYTES
    lib = hc.library()
    fake = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    fake[5] = fake[6] = None  # no prologue
    st = lib.hclrmix_run_noalloc(*fake, ctypes.byref(prob), ctypes.byref(attrs), None)
    assert st == hc.HCLRMIX_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in hc.hclrmix_last_error()
