"""GPU tests of the properties the block's contract rests on (onnxruntime PR
#33384, sections "Numerics contract" and "Testing"), beyond plain parity:

* a row's bits do not depend on the slot it takes in a matrix-core tile or on
  its neighbour rows: rows rolled and reversed across tile boundaries give the
  bits of a 2100-row reference;
* the up gate's sigmoid of every finite T value, through every path (and the
  bf16 lookup table of the many-row up kernel), against the oracle, in a
  wiring where pre_output equals g;
* ScaledSiLU of every finite T value of down, read back as hidden from the
  workspace, against the oracle's trace;
* hidden (the first rounding point after the down reduction) against the
  oracle's trace on sampled rows of the workloads;
* a workspace whose scratch starts as NaN gives the bits of a zeroed one;
* the same for a shape the matrix-core paths run zero-padded (slots, hidden,
  NaN scratch);
* the graph that bench.py times (96 chained calls over distinct weights, one
  shared workspace) replays to the bits of an eager chain of plain calls.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import hyper_connection_rank_amd as hc
import oracle
import synth
from _parity import NAMES, args_of, gpu_run
from _util import ulp_dist, ulp_of

pytestmark = pytest.mark.gpu

# The five workloads, and a shape that the matrix-core paths run zero-padded
# (H 2056 -> 2080, R 328 -> 352; the hidden size of the onnxruntime page's
# "Testing" shapes), whose hidden comes back through the output copy.
W = dict(synth.WORKLOADS)
W["padded_bf16"] = synth.Workload(1330, "padded_bf16", 600, 4, 2056, 328, "bf16", True, epsilon=1e-6,
                                  reduction_scale=0.25, silu_alpha=0.25, gate_div=4.0, gate_mul=2.0)
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _bits(x):
    return x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32)


# ----------------------------------------------------------------------------- slots and neighbours

def _perms(n: int, pool: int):
    """Row index sets of size n taken from a pool of `pool` rows: the prefix
    rolled by 1, 5 and 77 rows (row r lands in slot r - shift) and reversed."""
    base = np.arange(n)
    out = {f"roll{s}": (base + s) % pool for s in (1, 5, 77)}
    out["reversed"] = base[::-1].copy()
    return out


@pytest.mark.parametrize("wname", ["decode_bf16", "wide_f16", "padded_bf16"])
def test_row_bits_independent_of_slot_and_neighbours(wname):
    """Every row keeps its bits when it moves to another slot of the 16-row
    decode tile, the 128-row down tile and the 32-row up chunk, with other
    rows around it: subsets of 7, 16, 40, 600 and 2100 rows, rolled and
    reversed, on auto, decode and prefill, against one 2100-row prefill call
    (un-permuted, compared bitwise)."""
    w = W[wname]
    pool_n = 2100
    pool = synth.block_inputs(w, rows=pool_n)
    ref = gpu_run(pool, w.attrs(), path="prefill")
    acts = ("streams", "prev_block_output", "prev_post_gate")
    checked = 0
    for rows in (7, 16, 40, 600, 2100):
        for kind, idx in _perms(rows, pool_n).items():
            it = torch.from_numpy(idx)
            t = {k: (v.index_select(0, it).contiguous() if k in acts else v) for k, v in pool.items()}
            for path in ("auto", "decode", "prefill"):
                if path == "decode" and rows > hc.DECODE_MAX_ROWS:
                    continue
                print(f"[slots] {wname} rows={rows} {kind} path={path}", flush=True)
                out = gpu_run(t, w.attrs(), path=path)
                for name, x, y in zip(("pre_output", "post_gate", "streams_out"), out, ref):
                    assert torch.equal(_bits(x), _bits(y.index_select(0, it))), (rows, kind, path, name)
                checked += 1
    print(f"[slots] {wname}: {checked} permuted calls bit-identical to the reference", flush=True)


# ----------------------------------------------------------------------------- sigmoid and ScaledSiLU wiring

def _finite_values(dt: torch.dtype) -> torch.Tensor:
    """Every finite value of a 16-bit type, in bit order (+0 .. max, -0 .. -max)."""
    top = 0x7F80 if dt == torch.bfloat16 else 0x7C00  # first infinity pattern
    pos = torch.arange(0, top, dtype=torch.int32)
    bits = torch.cat([pos, pos | 0x8000]).to(torch.int16)
    return bits.view(dt)


def _gate_sweep_inputs(dt, values: torch.Tensor, rows: int):
    """C = 4, H = 2560, R = 320, no prologue, eps 0, rs 1/4, silu_alpha 64.
    streams = 1 and norm_scale = 1 make hn = 1 everywhere (every branch's mean
    square is 1). down_weight is zero except [0, 0] = 1, so down = (1, 0, ...)
    and hidden = (1, 0, ...) exactly (sigmoid(64) rounds to 1; ScaledSiLU(0) =
    0). up_weight's row 0 holds value v_h at column c*H + h of every branch c
    (its other rows are arbitrary: they meet hidden = 0), so up = v_h and
    pre_output[h] = rT(1/4 * 4 g) = g = rT(sigmoid(v_h)). inject_weight = 0."""
    C, H, R = 4, 2560, 320
    K = C * H
    v = torch.zeros(H, dtype=dt)
    v[: values.numel()] = values
    gen = torch.Generator().manual_seed(5)
    t = {
        "streams": torch.ones(rows, K, dtype=dt),
        "norm_scale": torch.ones(K, dtype=dt),
        "down_weight": torch.zeros(K, R, dtype=dt),
        "up_weight": torch.randn(R, K, generator=gen).to(dt),
        "inject_weight": torch.zeros(K, C, dtype=dt),
    }
    t["down_weight"][0, 0] = 1.0
    t["up_weight"][0] = v.repeat(C)
    attrs = dict(num_branches=C, epsilon=0.0, reduction_scale=0.25, silu_alpha=64.0, gate_div=1.0, gate_mul=1.0)
    return t, attrs


GATE_PATHS = [("decode", 1), ("prefill", 40), ("prefill", 520), ("generic", 1)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_up_gate_sigmoid_every_finite_value(dtype):
    """g = rT(sigmoid(v)) for every finite T value v, on the decode path, the
    prefill path with the plain up kernel (40 rows) and, for bf16, with the
    many-row up kernel and its sigmoid table (520 rows), and the generic path:
    within 1 ulp of the oracle (whose sigmoid divides by 1 + expf(-v)), and the
    same bits on every path."""
    dt = TDT[dtype]
    vals = _finite_values(dt)
    H = 2560
    worst = {}
    for i0 in range(0, vals.numel(), H):
        chunk = vals[i0:i0 + H]
        t1, attrs = _gate_sweep_inputs(dt, chunk, 1)
        o = oracle.run(*args_of(t1), **attrs)[0][0, : chunk.numel()]
        assert torch.equal(o.float(), o.float()), "oracle produced NaN"
        per_path = {}
        for path, rows in GATE_PATHS:
            if rows == 520 and dtype != "bf16":
                continue
            t, _ = _gate_sweep_inputs(dt, chunk, rows)
            pre = gpu_run(t, attrs, path=path, want_streams_out=False)[0]
            g = pre[:, : chunk.numel()]
            assert torch.equal(_bits(g), _bits(g[:1].expand_as(g))), (path, rows, "rows differ")
            d = ulp_dist(g[0].contiguous(), o.contiguous())
            key = f"{path}/{rows}"
            n_off = int((d != 0).sum())
            w_ = worst.setdefault(key, [0, 0])
            w_[0] = max(w_[0], int(d.max()))
            w_[1] += n_off
            assert int(d.max()) <= 1, (key, i0, int(d.max()))
            per_path[key] = g[0]
        first = next(iter(per_path.values()))
        for key, g in per_path.items():
            assert torch.equal(_bits(g), _bits(first)), (key, i0, "paths differ")
    print(f"[gate sweep {dtype}] {vals.numel()} values; per path (max ulp, values off by 1 ulp): {worst}",
          flush=True)


def _silu_sweep_inputs(dt, values: torch.Tensor, rows: int, alpha: float):
    """C = 4, H = 4096, R = 320, no prologue, eps 0. Row r: branch 0 of streams
    is one-hot at feature r (value 1), branches 1..3 are all 1; norm_scale is
    1/64 on branch 0 and 1 elsewhere. Branch 0's root mean square is then
    exactly 1/64, so hn = 1 at feature r and 0 at the other features of
    branch 0, and hn = 1 on branches 1..3, whose down_weight rows are zero. So
    down of row r = down_weight[r, :] exactly: rows r < `rows` of down_weight
    carry the swept values, and hidden = ScaledSiLU(value)."""
    C, H, R = 4, 4096, 320
    K = C * H
    n = rows * R
    v = torch.zeros(n, dtype=dt)
    v[: values.numel()] = values
    s = torch.ones(rows, K, dtype=dt)
    s[:, :H] = 0.0
    s[torch.arange(rows), torch.arange(rows)] = 1.0
    ns = torch.ones(K, dtype=dt)
    ns[:H] = 1.0 / 64.0
    wd = torch.zeros(K, R, dtype=dt)
    wd[:rows] = v.view(rows, R)
    gen = torch.Generator().manual_seed(6)
    t = {"streams": s, "norm_scale": ns, "down_weight": wd,
         "up_weight": (0.05 * torch.randn(R, K, generator=gen)).to(dt),
         "inject_weight": torch.zeros(K, C, dtype=dt)}
    attrs = dict(num_branches=C, epsilon=0.0, reduction_scale=1.0, silu_alpha=alpha, gate_div=1.0, gate_mul=1.0)
    return t, attrs


def _gpu_hidden(t, attrs, path):
    """Run one block and return hidden [rows, R] read from the workspace."""
    g = {k: v.cuda() for k, v in t.items()}
    rows, K = g["streams"].shape
    R = g["up_weight"].shape[0]
    dt = g["streams"].dtype
    a = hc.make_attrs(**attrs)
    prob = hc.make_problem(rows, K, R, hc.dtype_code(dt), "prev_block_output" in g, path)
    ws = hc.new_workspace(prob, a, "cuda")
    hc.block(*args_of(g), **attrs, path=path, workspace=ws)
    torch.cuda.synchronize()
    off = hc.hclrmix_hidden_offset(prob, a)
    es = 4 if dt == torch.float32 else 2
    raw = ws[off: off + rows * R * es].cpu()
    return raw.view(dt).view(rows, R)


def _oracle_hidden_rows(t, attrs, rows):
    out = []
    for r in rows:
        one = {k: (v[r:r + 1].contiguous() if k in ("streams", "prev_block_output", "prev_post_gate") else v)
               for k, v in t.items()}
        tr = oracle.trace(*args_of(one), row=0, **attrs)
        out.append(tr["hidden"])
    return torch.stack(out)


@pytest.mark.parametrize("alpha", [0.25, 1.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_scaled_silu_every_finite_value(dtype, alpha):
    """hidden = ScaledSiLU(down) for every finite T value of down (Z, SG and
    hidden rounded to T), read from the workspace, on the decode path (16 rows
    a call), the prefill path and the generic path (all rows in one call):
    within 1 ulp of the oracle's trace and the same bits on every path."""
    dt = TDT[dtype]
    vals = _finite_values(dt)
    R = 320
    rows_all = (vals.numel() + R - 1) // R
    t, attrs = _silu_sweep_inputs(dt, vals, rows_all, alpha)
    ora = _oracle_hidden_rows(t, attrs, range(rows_all))              # fp32 holding T values
    ora_t = ora.to(dt)
    pre = _gpu_hidden(t, attrs, "prefill")
    gen = _gpu_hidden(t, attrs, "generic")
    dec = []
    for r0 in range(0, rows_all, hc.DECODE_MAX_ROWS):
        r1 = min(rows_all, r0 + hc.DECODE_MAX_ROWS)
        sub = dict(t)
        # keep the one-hot positions: row r of the subset must still be row r0 + r of the sweep
        s = t["streams"][r0:r1].contiguous()
        sub["streams"] = s
        dec.append(_gpu_hidden(sub, attrs, "decode"))
    dec = torch.cat(dec)
    for name, x in (("decode", dec), ("prefill", pre), ("generic", gen)):
        d = ulp_dist(x.contiguous(), ora_t.contiguous())
        print(f"[silu sweep {dtype} alpha={alpha}] {name}: {vals.numel()} values, max ulp {int(d.max())}, "
              f"off by 1 ulp {int((d != 0).sum())}", flush=True)
        assert int(d.max()) <= 1, name
    assert torch.equal(_bits(dec), _bits(pre)) and torch.equal(_bits(gen), _bits(pre))


# ----------------------------------------------------------------------------- hidden against the trace

@pytest.mark.parametrize("wname,rows_to_check", [
    ("tiny_f32", [0, 1]), ("decode_bf16", [0]), ("prefill_bf16", [0, 4095, 8191]), ("wide_f16", [0, 37, 63]),
    ("padded_bf16", [0, 17, 599]),
])
def test_hidden_step_against_oracle_trace(wname, rows_to_check):
    """The first rounding point after the down reduction, hidden [rows, R],
    against the oracle's trace of the same rows: within 2 ulp of T, or (a sum
    that cancels) within 2 ulp of the magnitude sum_k |hn_k * Wd[k, n]|
    (from the trace's hn); fp32 within 1e-5 relative to that magnitude."""
    w = W[wname]
    t = synth.block_inputs(w)
    path = "auto"
    hid = _gpu_hidden(t, w.attrs(), path)
    wd = t["down_weight"].double()
    n_rejudged = 0
    for r in rows_to_check:
        one = {k: (v[r:r + 1].contiguous() if k in ("streams", "prev_block_output", "prev_post_gate") else v)
               for k, v in t.items()}
        tr = oracle.trace(*args_of(one), row=0, **w.attrs())
        mag = tr["hn"].double().abs() @ wd.abs()
        g, o = hid[r], tr["hidden"].to(hid.dtype)
        if hid.dtype == torch.float32:
            err = (g.double() - o.double()).abs()
            assert bool((err <= 1e-5 * torch.maximum(o.double().abs(), mag)).all()), (wname, r)
            continue
        d = ulp_dist(g.contiguous(), o.contiguous())
        off = d > 2
        ok = (g.double() - o.double()).abs() <= 2 * ulp_of(torch.maximum(mag, o.double().abs()), hid.dtype)
        assert bool((~off | ok).all()), (wname, r, int(d.max()))
        n_rejudged += int(off.sum())
        print(f"[hidden {wname}] row {r}: exact {(d == 0).float().mean().item():.4%}, max ulp {int(d.max())}, "
              f"re-judged {int(off.sum())}", flush=True)
    # measured: at most 1.1 % of the sampled hidden values (wide fp16) need the re-judge
    assert n_rejudged <= max(2, 3 * len(rows_to_check) * w.R // 100), n_rejudged


# ----------------------------------------------------------------------------- NaN-poisoned scratch

@pytest.mark.parametrize("path,rows,wname", [("decode", 3, "decode_bf16"), ("prefill", 40, "decode_bf16"),
                                            ("prefill", 600, "decode_bf16"), ("prefill", 64, "wide_f16"),
                                            ("generic", 5, "decode_bf16"), ("generic", 2, "tiny_f32"),
                                            ("decode", 3, "padded_bf16"), ("prefill", 40, "padded_bf16"),
                                            ("prefill", 600, "padded_bf16")])
def test_scratch_poisoned_with_nan(path, rows, wname):
    """Every byte of the workspace past the counter prefix (which must be zero
    before first use) set to 0xFF, a NaN in every float type: a kernel that
    read scratch it had not written first would carry NaN into an output. The
    outputs equal those of a zeroed workspace, bit for bit, twice in a row."""
    w = W[wname].replace(rows=rows)
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    a = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(rows, w.K, w.R, hc.dtype_code(t["streams"].dtype), w.has_prologue, path)
    clean = hc.block(*args_of(t), **w.attrs(), path=path)
    ws = hc.new_workspace(prob, a, "cuda")
    ws[4096:] = 0xFF
    for _ in range(2):
        got = hc.block(*args_of(t), **w.attrs(), path=path, workspace=ws)
        torch.cuda.synchronize()
        for x, y in zip(got, clean):
            assert not torch.isnan(x).any()
            assert torch.equal(_bits(x.cpu()), _bits(y.cpu())), (path, rows)


# ----------------------------------------------------------------------------- the timed graph

def test_benchmark_graph_of_chained_calls_matches_eager_chain():
    """The configuration bench.py times: 96 hclrmix_run_chained calls (rows 1,
    distinct seeded weights per block, each call given the next block's down
    and inject weights), one shared workspace, outputs ping-ponged between two
    buffer sets, captured as one HIP graph. Every replay (with eager work in
    between) ends with the bits of an eager chain of plain hclrmix_run calls,
    each on a fresh workspace."""
    w = W["decode_bf16"]
    nb = 96
    dt = torch.bfloat16
    weights = [{k: v.cuda() for k, v in synth.block_inputs(w, b, with_acts=False).items()} for b in range(nb)]
    acts0 = {k: v.cuda() for k, v in synth.block_inputs(w, 0, with_weights=False).items()}
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(1, w.K, w.R, hc.HCLRMIX_BF16, True)

    # eager reference: plain calls, a fresh workspace per block
    s, p, g = acts0["streams"], acts0["prev_block_output"], acts0["prev_post_gate"]
    for b in range(nb):
        W_ = weights[b]
        o = [torch.empty(1, w.H, dtype=dt, device="cuda"), torch.empty(1, w.C, dtype=dt, device="cuda"),
             torch.empty(1, w.K, dtype=dt, device="cuda")]
        hc.hclrmix_run(s, W_["norm_scale"], W_["down_weight"], W_["up_weight"], W_["inject_weight"], p, g,
                       o[0], o[1], o[2], hc.new_workspace(prob, attrs, "cuda"), prob, attrs)
        s, p, g = o[2], o[0], o[1]
    torch.cuda.synchronize()
    ref = [p.clone(), g.clone(), s.clone()]

    ws = hc.new_workspace(prob, attrs, "cuda")
    sets = [dict(streams=torch.empty(1, w.K, dtype=dt, device="cuda"), pre=torch.empty(1, w.H, dtype=dt, device="cuda"),
                 post=torch.empty(1, w.C, dtype=dt, device="cuda")) for _ in range(2)]

    def reset():
        sets[0]["streams"].copy_(acts0["streams"])
        sets[0]["pre"].copy_(acts0["prev_block_output"])
        sets[0]["post"].copy_(acts0["prev_post_gate"])

    def chain():
        for b in range(nb):
            i, o = sets[b % 2], sets[(b + 1) % 2]
            W_, N = weights[b], weights[(b + 1) % nb]
            hc.hclrmix_run_chained(i["streams"], W_["norm_scale"], W_["down_weight"], W_["up_weight"],
                                   W_["inject_weight"], i["pre"], i["post"], o["pre"], o["post"], o["streams"],
                                   ws, prob, attrs, next_down_weight=N["down_weight"],
                                   next_inject_weight=N["inject_weight"])

    reset()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        chain()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    last = sets[nb % 2]
    for x, y in zip((last["pre"], last["post"], last["streams"]), ref):
        assert torch.equal(_bits(x), _bits(y)), "eager chained calls"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip((last["pre"], last["post"], last["streams"]), ref):
            assert torch.equal(_bits(x), _bits(y)), f"replay {rep}"
        z = torch.randn(4096, device="cuda")
        (z * 3).sum().item()
    print(f"[timed graph] {nb} chained blocks: every replay bit-identical to the eager plain chain", flush=True)
