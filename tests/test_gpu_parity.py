"""GPU parity: the HIP library against the CPU oracle on the same seeded
inputs, through the C-ABI (Python binding), for the five workloads and a
sweep of small shapes; plus bitwise determinism, batch invariance across row
counts and paths, HIP-graph replay and guard canaries."""
from __future__ import annotations

import pytest
import torch

import hyper_connection_rank_amd as hc
import synth
from _parity import args_of, assert_parity, gpu_run, judge_block, oracle_run

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _small(C, H, R, rows, dtype, prologue=True, wid=500, **attrs):
    base = dict(epsilon=1e-6, reduction_scale=0.25, silu_alpha=0.25, gate_div=4.0, gate_mul=2.0)
    base.update(attrs)
    return synth.Workload(wid, "sweep", rows, C, H, R, dtype, prologue, **base)


def _check(w, path="auto", rows=None, block=0, want_streams_out=True, label=None):
    t = synth.block_inputs(w, block, rows=rows)
    g = gpu_run(t, w.attrs(), path=path, want_streams_out=want_streams_out)
    o = oracle_run(t, w.attrs())
    assert_parity(judge_block(g, o, want_streams_out), label or f"{w.name} path={path}")
    return t, g, o


# ----------------------------------------------------------------------------- the five workloads

def test_tiny_fp32_block():
    _check(W["tiny_f32"])


@pytest.mark.parametrize("path", ["auto", "prefill", "generic"])
def test_decode_block_bf16(path):
    _check(W["decode_bf16"], path=path)


def test_prefill_block_bf16_full():
    _check(W["prefill_bf16"])


@pytest.mark.parametrize("path", ["auto", "generic"])
def test_wide_block_fp16(path):
    _check(W["wide_f16"], path=path)


def test_wide_block_fp16_decode_rows():
    """The wide fp16 shape through the decode path (its 16-row limit)."""
    _check(W["wide_f16"].replace(rows=16), path="decode")


def test_decode_chain_bf16_teacher_forced():
    """96 chained blocks, rows = 8, each with its own seeded weights. Block b
    takes block b-1's streams_out, pre_output and post_gate (GPU values); the
    oracle gets the same inputs for every block (teacher forcing)."""
    w = W["decode_chain_bf16"]
    acts = synth.block_inputs(w, 0, with_weights=False)
    worst = []
    for b in range(w.blocks):
        t = dict(synth.block_inputs(w, b, with_acts=False))
        t.update(acts)
        g = gpu_run(t, w.attrs())
        o = oracle_run(t, w.attrs())
        js = judge_block(g, o)
        if any(j.bad for j in js) or b in (0, w.blocks - 1):
            assert_parity(js, f"decode chain bf16 block {b}")
        worst.append(max(j.max_ulp for j in js))
        acts = {"streams": g[2], "prev_block_output": g[0], "prev_post_gate": g[1]}
    print(f"chain: max ulp per block {worst}", flush=True)


# ----------------------------------------------------------------------------- shape sweep

# (2, 1184, 32, 11): 1184 = 32 x 37 gives 37 slices of 32 features per branch,
# so a branch has 407 slice partial rows at 11 rows, more than the decode
# reduction stages in LDS at once (it takes them through registers).
# (8, 2560, 320, 20): 320 up units of 64 features, more than the compute
# units, so the few-row up kernel's workgroups take two each.
SWEEP = [
    (1, 32, 32, 1), (2, 64, 32, 5), (3, 96, 64, 16), (4, 256, 32, 17), (8, 64, 64, 33),
    (4, 512, 96, 3), (2, 288, 128, 70), (1, 2080, 32, 9), (4, 64, 512, 20), (2, 1184, 32, 11),
    (8, 2560, 320, 20), (4, 640, 96, 130), (2, 128, 64, 449),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("C,H,R,rows", SWEEP)
@pytest.mark.parametrize("prologue", [True, False])
def test_matrix_core_sweep(dtype, C, H, R, rows, prologue):
    w = _small(C, H, R, rows, dtype, prologue, wid=600 + C * 7 + H + R)
    for path in ("decode", "prefill"):
        if path == "decode" and rows > hc.DECODE_MAX_ROWS:
            continue
        _check(w, path=path)


@pytest.mark.parametrize("R,rows", [(320, 1800), (96, 1300)])
def test_prefill_units_cross_column_groups(R, rows):
    """More (column group, 512-row block) units than workgroups: a workgroup
    walks several units, changes column group between them and meets the
    partial last row block; R < 320 runs the zero-padded chain."""
    w = _small(4, 2560, R, rows, "bf16", True, wid=900 + R)
    _check(w, path="prefill")


@pytest.mark.parametrize("C,H,R,rows", [(1, 256, 64, 600), (2, 192, 96, 530), (8, 64, 320, 520),
                                        (8, 96, 160, 700), (4, 128, 320, 640)])
def test_prefill_up_kernel_every_branch_count(C, H, R, rows):
    """The bf16 up kernel above 512 rows for each branch count it is built
    for, full and zero-padded rank, with streams_out given (hn rebuilt from
    it) and not given (S rebuilt from the prologue inputs): each against the
    oracle, and the two bitwise equal."""
    w = _small(C, H, R, rows, "bf16", True, wid=950 + C)
    _, a, _ = _check(w, path="prefill", label=f"up kernel C={C} H={H} R={R} rows={rows} streams_out")
    _, b, _ = _check(w, path="prefill", want_streams_out=False,
                     label=f"up kernel C={C} H={H} R={R} rows={rows} no streams_out")
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("C,H,R,rows", [(1, 8, 8, 3), (3, 33, 16, 4), (4, 48, 24, 2), (2, 100, 40, 5),
                                         (16, 32, 32, 2), (4, 2560, 320, 2)])
def test_generic_sweep(dtype, C, H, R, rows):
    w = _small(C, H, R, rows, dtype, True, wid=700 + C + H + R)
    _check(w, path="generic")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_non_default_attributes(dtype):
    w = _small(4, 128, 64, 6, dtype, True, wid=800, epsilon=1e-3, reduction_scale=0.75,
               silu_alpha=1.5, gate_div=0.5, gate_mul=3.0)
    for path in ("decode", "prefill", "generic"):
        _check(w, path=path)


@pytest.mark.parametrize("rows", [5, 100])
def test_streams_out_optional_same_bits(rows):
    w = W["decode_bf16"].replace(rows=rows)
    t = synth.block_inputs(w)
    for path in (("decode", "prefill") if rows <= hc.DECODE_MAX_ROWS else ("prefill",)):
        a = gpu_run(t, w.attrs(), path=path, want_streams_out=True)
        b = gpu_run(t, w.attrs(), path=path, want_streams_out=False)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and b[2] is None


# ----------------------------------------------------------------------------- determinism

def _bits(x):
    return x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32)


@pytest.mark.parametrize("wname", ["decode_bf16", "wide_f16"])
def test_batch_invariance_across_rows_and_paths(wname):
    """Row r gives the same bits at every row count and on both matrix-core
    paths (onnxruntime PR #33384, "Numerics contract": per-row results do not
    depend on the row count).
    The reference is 2100 rows of prefill (a branch per down workgroup; the
    bf16 up kernel with the transposed weights); the subsets cover decode,
    prefill's slice mode with either down kernel (the few-row one up to 128
    rows for the 4x2560 shape) and each up kernel (up to 128 rows: the
    per-branch one, in two row blocks of 64 from 65 rows; 129 to 512: the
    plain one; 513 and 600: the bf16 one with transposed weights, or the
    plain one for fp16)."""
    w = W[wname]
    pool = synth.block_inputs(w, rows=2100)
    ref = gpu_run(pool, w.attrs(), path="prefill")
    for rows in (1, 2, 3, 7, 8, 16, 17, 33, 40, 64, 65, 100, 128, 449, 512, 513, 600):
        t = {k: (v[:rows].contiguous() if k in ("streams", "prev_block_output", "prev_post_gate") else v)
             for k, v in pool.items()}
        for path in ("auto", "decode", "prefill"):
            if path == "decode" and rows > hc.DECODE_MAX_ROWS:
                continue
            out = gpu_run(t, w.attrs(), path=path)
            for x, y in zip(out, ref):
                assert torch.equal(_bits(x), _bits(y[:rows])), (rows, path)


@pytest.mark.parametrize("C,H,R,dtype,prologue", [(4, 64, 16, "f32", True), (3, 33, 16, "bf16", True),
                                                   (2, 100, 40, "f16", False), (8, 96, 32, "f32", True)])
def test_generic_one_workgroup_form_same_bits(C, H, R, dtype, prologue):
    """Small problems run the generic path as one workgroup (all four steps in
    one launch); the rows of a 40-row call, which takes the four-kernel form,
    give the same bits, the tiny fp32 workload's shape included."""
    w = _small(C, H, R, 40, dtype, prologue, wid=980 + C + H)
    pool = synth.block_inputs(w, rows=40)
    ref = gpu_run(pool, w.attrs(), path="generic")
    for rows in (1, 2, 5, 8, 16):
        t = {k: (v[:rows].contiguous() if k in ("streams", "prev_block_output", "prev_post_gate") else v)
             for k, v in pool.items()}
        out = gpu_run(t, w.attrs(), path="generic")
        for x, y in zip(out, ref):
            assert torch.equal(_bits(x), _bits(y[:rows])), (rows, C, H, R, dtype)


def test_one_workspace_for_every_path():
    """One zero-filled workspace, sized for the largest call, shared by
    decode, prefill and generic calls in turn: the decode arrival counters
    (which must stay zero between calls) survive the other paths' use of the
    workspace, and every call matches the same call on a fresh workspace."""
    wd = W["decode_bf16"]
    small = synth.block_inputs(wd, rows=3)
    big = synth.block_inputs(wd, rows=40)
    attrs = wd.attrs()
    calls = [(small, "decode", 3), (big, "prefill", 40), (small, "decode", 3), (big, "generic", 40),
             (small, "decode", 3)]
    a = hc.make_attrs(**attrs)
    size = max(hc.hclrmix_workspace_size(hc.make_problem(n, wd.K, wd.R, hc.HCLRMIX_BF16, True, p), a)
               for _, p, n in calls)
    shared = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for t, path, n in calls:
        g = {k: v.cuda() for k, v in t.items()}
        got = hc.block(*args_of(g), **attrs, path=path, workspace=shared)
        fresh = hc.block(*args_of(g), **attrs, path=path)
        torch.cuda.synchronize()
        for x, y in zip(got, fresh):
            assert torch.equal(_bits(x.cpu()), _bits(y.cpu())), path


def test_reruns_are_bitwise_equal():
    w = W["decode_bf16"].replace(rows=9)
    t = synth.block_inputs(w)
    for path in ("decode", "prefill", "generic"):
        a = gpu_run(t, w.attrs(), path=path)
        b = gpu_run(t, w.attrs(), path=path)
        for x, y in zip(a, b):
            assert torch.equal(_bits(x), _bits(y))


def test_zero_rows():
    w = W["decode_bf16"].replace(rows=0)
    t = synth.block_inputs(w, rows=0)
    pre, post, so = gpu_run(t, w.attrs())
    assert pre.shape == (0, 2560) and post.shape == (0, 4) and so.shape == (0, 10240)


@pytest.mark.parametrize("path", ["decode", "prefill", "generic"])
def test_guard_canaries_untouched(path):
    """Outputs are written only inside their [rows, cols] extent: NaN-filled
    guard rows after each output stay NaN."""
    w = W["decode_bf16"].replace(rows=3)
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    dt = t["streams"].dtype
    pre = torch.full((4, 2560), float("nan"), dtype=dt, device="cuda")
    post = torch.full((4, 4), float("nan"), dtype=dt, device="cuda")
    so = torch.full((4, 10240), float("nan"), dtype=dt, device="cuda")
    hc.block(*args_of(t), **w.attrs(), path=path, out=(pre[:3], post[:3], so[:3]))
    torch.cuda.synchronize()
    assert torch.isnan(pre[3]).all() and torch.isnan(post[3]).all() and torch.isnan(so[3]).all()
    assert not torch.isnan(pre[:3]).any() and not torch.isnan(post[:3]).any()


@pytest.mark.parametrize("path,rows", [("decode", 1), ("decode", 4), ("prefill", 4), ("prefill", 600)])
def test_hip_graph_replay_matches_eager(path, rows):
    """A captured call replays bit-identically to the eager call, replay after
    replay, with eager work in between."""
    w = W["decode_bf16"].replace(rows=rows)
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    dt = t["streams"].dtype
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(rows, w.K, w.R, hc.dtype_code(dt), True, path)
    ws = hc.new_workspace(prob, attrs, "cuda")
    outs = [torch.empty(rows, w.H, dtype=dt, device="cuda"), torch.empty(rows, w.C, dtype=dt, device="cuda"),
            torch.empty(rows, w.K, dtype=dt, device="cuda")]

    def call():
        hc.hclrmix_run(*args_of(t), *outs, ws, prob, attrs)

    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(_bits(o), _bits(e)), f"replay {i}"
        x = torch.randn(1024, device="cuda")  # unrelated eager work between replays
        (x * 2).sum().item()


@pytest.mark.parametrize("path,rows,nk", [("decode", 1, 2), ("decode", 12, 2), ("decode", 13, 3), ("prefill", 5, 5),
                                         ("prefill", 100, 5),
                                         ("prefill", 600, 5), ("generic", 5, 4)])
def test_timed_entry_point_same_bits(path, rows, nk):
    """hclrmix_run_timed launches the same kernels as hclrmix_run (bitwise
    equal outputs), reports their count and stamps a positive interval on
    each kernel's own start/stop event pair."""
    w = W["decode_bf16"].replace(rows=rows)
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    dt = t["streams"].dtype
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(rows, w.K, w.R, hc.dtype_code(dt), True, path)
    ws = hc.new_workspace(prob, attrs, "cuda")

    def outs():
        return [torch.empty(rows, w.H, dtype=dt, device="cuda"), torch.empty(rows, w.C, dtype=dt, device="cuda"),
                torch.empty(rows, w.K, dtype=dt, device="cuda")]

    ref, got = outs(), outs()
    hc.hclrmix_run(*args_of(t), *ref, ws, prob, attrs)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * hc.MAX_KERNELS)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    k = hc.hclrmix_run_timed(*args_of(t), *got, ws, prob, attrs, [e.cuda_event for e in evs])
    torch.cuda.synchronize()
    assert k == nk
    for x, y in zip(ref, got):
        assert torch.equal(_bits(x), _bits(y))
    for i in range(k):
        assert evs[2 * i].elapsed_time(evs[2 * i + 1]) > 0.0


@pytest.mark.parametrize("path,rows", [("decode", 1), ("decode", 5), ("prefill", 5), ("generic", 3)])
def test_chained_call_same_bits(path, rows):
    """hclrmix_run_chained (next block's weights prefetched while this block's
    last kernel runs) gives the bits of hclrmix_run, over a short chain of
    blocks with distinct weights, untimed and timed."""
    w = W["decode_bf16"].replace(rows=rows)
    nb = 4
    weights = [{k: v.cuda() for k, v in synth.block_inputs(w, b, with_acts=False).items()} for b in range(nb)]
    acts = {k: v.cuda() for k, v in synth.block_inputs(w, 0, with_weights=False).items()}
    dt = acts["streams"].dtype
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(rows, w.K, w.R, hc.dtype_code(dt), True, path)

    def run_chain(chained, timed=False):
        ws = hc.new_workspace(prob, attrs, "cuda")
        s, p, g = acts["streams"], acts["prev_block_output"], acts["prev_post_gate"]
        outs = []
        for b in range(nb):
            W_ = weights[b]
            nxt = weights[(b + 1) % nb]
            o = [torch.empty(rows, w.H, dtype=dt, device="cuda"), torch.empty(rows, w.C, dtype=dt, device="cuda"),
                 torch.empty(rows, w.K, dtype=dt, device="cuda")]
            args = (s, W_["norm_scale"], W_["down_weight"], W_["up_weight"], W_["inject_weight"], p, g,
                    o[0], o[1], o[2], ws, prob, attrs)
            if chained:
                evs = None
                if timed:
                    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * hc.MAX_KERNELS)]
                    for e in evs:
                        e.record()
                k = hc.hclrmix_run_chained(*args, next_down_weight=nxt["down_weight"],
                                           next_inject_weight=nxt["inject_weight"],
                                           events=None if evs is None else [e.cuda_event for e in evs])
                assert (k > 0) == timed
            else:
                hc.hclrmix_run(*args)
            outs.append(o)
            s, p, g = o[2], o[0], o[1]
        torch.cuda.synchronize()
        return outs

    ref = run_chain(False)
    for timed in (False, True):
        got = run_chain(True, timed)
        for b in range(nb):
            for x, y in zip(ref[b], got[b]):
                assert torch.equal(_bits(x), _bits(y)), (path, rows, timed, b)


# ----------------------------------------------------------------------------- irregular shapes
# The shape matrix of the onnxruntime page's tests (section "Testing"): branch
# counts 1, 2, 3, 8; hidden sizes that are not multiples of 8 or 32; ranks from
# 8 to 512; odd row counts; fp32 at any row count. Shapes outside the
# matrix-core envelope take the generic path (auto), the others one of the
# matrix-core paths.
IRREGULAR = [
    (1, 33, 8, 1, "bf16"), (2, 100, 24, 9, "bf16"), (3, 72, 40, 17, "f16"), (8, 40, 16, 3, "bf16"),
    (3, 4095, 8, 2, "bf16"), (8, 513, 512, 1, "f16"), (2, 2056, 320, 1, "bf16"), (4, 2056, 328, 5, "bf16"),
    (1, 4096, 512, 8, "f16"), (8, 4096, 512, 1, "bf16"), (3, 96, 96, 33, "bf16"), (2, 7, 8, 40, "f32"),
    (4, 2560, 320, 1, "f32"), (4, 2560, 320, 17, "f32"), (3, 33, 17, 6, "f32"), (8, 1000, 104, 2, "f16"),
]


@pytest.mark.parametrize("C,H,R,rows,dtype", IRREGULAR)
@pytest.mark.parametrize("prologue", [True, False])
def test_irregular_shape_matrix(C, H, R, rows, dtype, prologue):
    w = _small(C, H, R, rows, dtype, prologue, wid=1000 + C * 13 + H + R + rows)
    _check(w, path="auto")


# ----------------------------------------------------------------------------- zero-padded matrix-core runs
# 16-bit shapes whose H or R is not a multiple of 32 run the matrix-core
# kernels on copies zero-padded to the next multiples of 32 (one copy kernel
# before, one after): H and R multiples of 8 (the page's hidden 2056), not
# multiples of 8, one of the two aligned, the smallest rank.
PADDED = [(4, 2056, 328, "bf16"), (2, 2056, 320, "bf16"), (3, 72, 40, "f16"), (8, 40, 16, "bf16"),
          (1, 33, 8, "bf16"), (8, 1000, 104, "f16"), (2, 4095, 512, "bf16")]


@pytest.mark.parametrize("C,H,R,dtype", PADDED)
def test_padded_shapes_batch_invariant_across_rows_and_paths(C, H, R, dtype):
    """A zero-padded shape keeps the matrix-core paths' contract: 600 rows of
    prefill match the oracle, and every subset of rows, on auto, decode and
    prefill, gives the same bits as those rows of the 600-row call."""
    w = _small(C, H, R, 600, dtype, True, wid=1200 + C * 11 + H + R)
    pool = synth.block_inputs(w)
    print(f"[padded] C={C} H={H} R={R} {dtype}", flush=True)
    ref = gpu_run(pool, w.attrs(), path="prefill")
    assert_parity(judge_block(ref, oracle_run(pool, w.attrs()), True), f"padded C={C} H={H} R={R} 600 rows")
    for rows in (1, 5, 12, 16, 17, 40, 513):
        t = {k: (v[:rows].contiguous() if k in ("streams", "prev_block_output", "prev_post_gate") else v)
             for k, v in pool.items()}
        for path in ("auto", "decode", "prefill"):
            if path == "decode" and rows > hc.DECODE_MAX_ROWS:
                continue
            out = gpu_run(t, w.attrs(), path=path)
            for x, y in zip(out, ref):
                assert torch.equal(_bits(x), _bits(y[:rows])), (rows, path)


def _off16(x):
    """x's values at an address one element past a 16-byte boundary."""
    buf = torch.empty(x.numel() + 16, dtype=x.dtype, device=x.device)
    y = buf[1:1 + x.numel()].view(x.shape)
    y.copy_(x)
    return y


@pytest.mark.parametrize("path,rows", [("decode", 3), ("prefill", 40)])
def test_padded_shape_takes_element_aligned_tensors(path, rows):
    """A zero-padded problem's kernels read only its workspace, so its tensors
    need element alignment only: every tensor one element off 16 bytes gives
    the bits of the aligned call (an unpadded shape refuses such pointers)."""
    w = _small(3, 72, 40, rows, "bf16", True, wid=1300)
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    ref = hc.block(*args_of(t), **w.attrs(), path=path, want_streams_out=True)
    u = {k: _off16(v) for k, v in t.items()}
    outs = tuple(_off16(torch.zeros_like(o)) for o in ref)
    got = hc.block(*args_of(u), **w.attrs(), path=path, out=outs)
    torch.cuda.synchronize()
    for x, y in zip(ref, got):
        assert torch.equal(_bits(x.cpu()), _bits(y.cpu())), path
    v = _small(3, 64, 32, rows, "bf16", True, wid=1301)
    tv = {k: _off16(v_.cuda()) for k, v_ in synth.block_inputs(v).items()}
    with pytest.raises(hc.HclrmixError) as e:
        hc.block(*args_of(tv), **v.attrs(), path=path)
    assert e.value.status == hc.HCLRMIX_ERR_UNSUPPORTED


def _timed_count(w, t, path):
    """Kernels hclrmix_run_timed reports for workload w on inputs t."""
    dt = t["streams"].dtype
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(w.rows, w.K, w.R, hc.dtype_code(dt), True, path)
    outs = [torch.empty(w.rows, w.H, dtype=dt, device="cuda"), torch.empty(w.rows, w.C, dtype=dt, device="cuda"),
            torch.empty(w.rows, w.K, dtype=dt, device="cuda")]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * hc.MAX_KERNELS)]
    k = hc.hclrmix_run_timed(*args_of(t), *outs, hc.new_workspace(prob, attrs, "cuda"), prob, attrs,
                             [e.cuda_event for e in evs])
    torch.cuda.synchronize()
    return k


@pytest.mark.parametrize("path,rows", [("decode", 1), ("decode", 12), ("prefill", 5), ("prefill", 600)])
def test_padded_timed_and_graph_replay(path, rows):
    """The timed entry point brackets the two copy kernels too: two kernels
    more than the same path runs for the padded sizes (H 2080, R 352), and the
    untimed call's bits; a captured padded call replays bit-identically."""
    w = _small(4, 2056, 328, rows, "bf16", True, wid=1310)
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    dt = t["streams"].dtype
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(rows, w.K, w.R, hc.dtype_code(dt), True, path)
    ws = hc.new_workspace(prob, attrs, "cuda")

    def outs():
        return [torch.zeros(rows, w.H, dtype=dt, device="cuda"), torch.zeros(rows, w.C, dtype=dt, device="cuda"),
                torch.zeros(rows, w.K, dtype=dt, device="cuda")]

    ref, got = outs(), outs()
    hc.hclrmix_run(*args_of(t), *ref, ws, prob, attrs)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * hc.MAX_KERNELS)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    k = hc.hclrmix_run_timed(*args_of(t), *got, ws, prob, attrs, [e.cuda_event for e in evs])
    torch.cuda.synchronize()
    wp = _small(4, 2080, 352, rows, "bf16", True, wid=1311)
    assert k == _timed_count(wp, {n: v.cuda() for n, v in synth.block_inputs(wp).items()}, path) + 2
    for x, y in zip(ref, got):
        assert torch.equal(_bits(x), _bits(y))
    for i in range(k):
        assert evs[2 * i].elapsed_time(evs[2 * i + 1]) > 0.0
    graph_out = outs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        hc.hclrmix_run(*args_of(t), *graph_out, ws, prob, attrs)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hc.hclrmix_run(*args_of(t), *graph_out, ws, prob, attrs)
    for i in range(3):
        for o in graph_out:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(ref, graph_out):
            assert torch.equal(_bits(x), _bits(y)), f"replay {i}"


# ----------------------------------------------------------------------------- large tensors

def test_prefill_streams_beyond_4_gib():
    """streams (and streams_out) larger than 4 GiB: the prefill kernels'
    row-relative 32-bit offsets must not wrap. Rows on both sides of the 4 GiB
    byte offset, and the last row, match the oracle run on those rows alone
    (a row's outputs depend on its own inputs and the weights only)."""
    w = W["prefill_bf16"]
    K, H, C = w.K, w.H, w.C
    edge = (1 << 32) // (K * 2)  # first row that starts past 4 GiB
    rows = edge + 200
    small = synth.block_inputs(w, 0, rows=1)  # weights and norm_scale of the workload (seeded)
    gen = torch.Generator(device="cuda").manual_seed(20261202)
    dt = torch.bfloat16
    dev = {k: small[k].cuda() for k in ("norm_scale", "down_weight", "up_weight", "inject_weight")}
    dev["streams"] = torch.randn(rows, K, generator=gen, device="cuda", dtype=dt)
    dev["prev_block_output"] = torch.randn(rows, H, generator=gen, device="cuda", dtype=dt)
    dev["prev_post_gate"] = (2.0 * torch.rand(rows, C, generator=gen, device="cuda")).to(dt)
    assert dev["streams"].numel() * 2 > (1 << 32)
    print(f"[large] rows={rows} streams bytes={dev['streams'].numel() * 2}", flush=True)
    try:
        out = hc.block(*args_of(dev), **w.attrs(), want_streams_out=True, path="prefill")
        torch.cuda.synchronize()
        pick = torch.tensor([0, edge - 2, edge - 1, edge, edge + 1, rows - 1], device="cuda")
        g = tuple(o.index_select(0, pick).cpu() for o in out)
        t = {k: (v.index_select(0, pick).cpu() if k in ("streams", "prev_block_output", "prev_post_gate")
                 else v.cpu()) for k, v in dev.items()}
        del out
    finally:
        del dev
        torch.cuda.empty_cache()
    o = oracle_run(t, w.attrs())
    assert_parity(judge_block(g, o, True), "prefill beyond 4 GiB")
