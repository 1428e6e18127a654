"""hclrmix_run_noalloc (the entry point for callers that cannot allocate
device memory: its scratch is the library's static device array) against
hclrmix_run with a workspace: the same kernels on the same layout, so the
outputs must be bit-identical. Two calls in a row on each path, the second
with fewer rows, so the second call meets the first call's leftovers in the
shared array; then a problem whose scratch exceeds the array is refused."""
from __future__ import annotations

import pytest
import torch

import hyper_connection_rank_amd as hc
import synth

pytestmark = pytest.mark.gpu


# A shape the matrix-core paths run zero-padded (H 2056 -> 2080, R 328 -> 352):
# its scratch also holds the padded copies.
PADDED = synth.Workload(1320, "padded_bf16", 7, 4, 2056, 328, "bf16", True, epsilon=1e-6, reduction_scale=0.25,
                        silu_alpha=0.25, gate_div=4.0, gate_mul=2.0)


def _bits(x):
    return x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32)


def _outs(w, rows, dt):
    return [torch.empty(rows, w.H, dtype=dt, device="cuda"), torch.empty(rows, w.C, dtype=dt, device="cuda"),
            torch.empty(rows, w.K, dtype=dt, device="cuda")]


def _pair(w, rows, path, seed_block):
    t = {k: v.cuda() for k, v in synth.block_inputs(w, seed_block, rows=rows).items()}
    dt = t["streams"].dtype
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(rows, w.K, w.R, hc.dtype_code(dt), w.has_prologue, path)
    names = ("streams", "norm_scale", "down_weight", "up_weight", "inject_weight", "prev_block_output",
             "prev_post_gate")
    args = [t.get(n) for n in names]
    ref, got = _outs(w, rows, dt), _outs(w, rows, dt)
    hc.hclrmix_run(*args, *ref, hc.new_workspace(prob, attrs, "cuda"), prob, attrs)
    hc.hclrmix_run_noalloc(*args, *got, prob, attrs)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("path,wname,rows", [("decode", "decode_bf16", (9, 1)), ("decode", "wide_f16", (16, 3)),
                                             ("prefill", "decode_bf16", (40, 20)), ("prefill", "wide_f16", (17, 5)),
                                             ("generic", "decode_bf16", (5, 2)), ("generic", "tiny_f32", (2, 1)),
                                             ("decode", "padded_bf16", (7, 2)), ("prefill", "padded_bf16", (40, 17))])
def test_noalloc_matches_workspace_call(path, wname, rows):
    w = PADDED if wname == "padded_bf16" else synth.WORKLOADS[wname]
    for i, n in enumerate(rows):
        print(f"[noalloc] {path} {wname} rows={n} (call {i + 1})", flush=True)
        ref, got = _pair(w.replace(rows=n), n, path, seed_block=i)
        for name, x, y in zip(("pre_output", "post_gate", "streams_out"), ref, got):
            assert torch.equal(_bits(x), _bits(y)), (path, wname, n, name)


def test_noalloc_refuses_scratch_beyond_its_array():
    w = synth.WORKLOADS["prefill_bf16"]
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(w.rows, w.K, w.R, hc.HCLRMIX_BF16, True)
    assert hc.hclrmix_workspace_size(prob, attrs) > hc.NOALLOC_SCRATCH_BYTES
    t = {k: v.cuda() for k, v in synth.block_inputs(w, rows=8).items()}
    names = ("streams", "norm_scale", "down_weight", "up_weight", "inject_weight", "prev_block_output",
             "prev_post_gate")
    # shapes of the 8192-row problem are only checked on the host: the call is refused before any launch
    with pytest.raises(hc.HclrmixError) as e:
        hc.hclrmix_run_noalloc(*[t.get(n) for n in names], *_outs(w, 8, torch.bfloat16), prob, attrs)
    assert e.value.status == hc.HCLRMIX_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in hc.hclrmix_last_error()
