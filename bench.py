#!/usr/bin/env python3
"""Benchmark of the HyperConnectionLowRankMix block on one MI355X.

Headline (one JSON line on stdout): microseconds per block and HBM GB/s at
rows = 1, bf16, 4 streams x 2560, rank 320, with the prologue -- the decode
block of onnxruntime PR #33384 ("Benchmark": a 96-block chain, HIP-graph
replay, distinct weights per block so they come from HBM). One step is one
replay of the 96-block chain; value = step time / 96. The 96 weight sets
(1.27 GB) are far larger than L2 + MALL (8 x 4 MB + 256 MB).

Also reported: the slope between 96- and 48-block graphs (the pages' method),
per-kernel durations from HIP events recorded between the kernels on the
stream they run on, the roofline of the dominant kernel, rows = 8192 prefill
TFLOP/s, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/block + HBM GB/s at rows=1 bf16 (4x2560,R=320); TFLOP/s at rows=8192"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD specification
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD specification

# Algorithmic bytes of the decode block at rows = 1 (C=4, H=2560, R=320, bf16):
# every input read once, every output written once.
DEC_DOWN_BYTES = 10240 * 320 * 2 + 10240 * 4 * 2 + 10240 * 2 + 10240 * 2 + 2560 * 2 + 4 * 2 + 10240 * 2
DEC_UP_BYTES = 320 * 10240 * 2 + 2560 * 2
DEC_POST_BYTES = 4 * 2
DEC_BLOCK_BYTES = DEC_DOWN_BYTES + DEC_UP_BYTES + DEC_POST_BYTES   # 13,260,816
PF_ROWS = 8192
PF_FLOP = 2 * PF_ROWS * 10240 * (320 + 320 + 4)                   # 108.045 GFLOP
PF_BYTES = (PF_ROWS * 10240 * 2 * 2 + PF_ROWS * 2560 * 2 * 2 + PF_ROWS * 4 * 2 * 2
            + 10240 * 320 * 2 * 2 + 10240 * 4 * 2 + 10240 * 2)     # 432,771,072
# The prefill block's own roofline: min(matrix peak, FLOP/byte x HBM peak) = 1,997 TFLOP/s.
PF_ROOF_TFLOPS = min(MFMA_BF16_PEAK_TFLOPS, PF_FLOP / PF_BYTES * HBM_PEAK_GBPS / 1000.0)

# Kernels of one call, in launch order: decode, and prefill at rows = 8192
# (bf16: the branch reduction and the up kernel's preparation share one
# launch, then the many-row up kernel k_pf_up2).
KERNELS = {1: ("hc_down", "hc_uppre"), 2: ("pf_rms", "pf_down", "reduce_prep", "pf_up2")}
MAX_KERNELS = 7  # most kernels one hclrmix_run launches


# HBM traffic per launch comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE
# summaries committed under profiles/ (counters are taken in their own runs,
# never inside this timed process). Each summary records a SHA-256 over the
# kernel's sources; a kernel edited since its counters were taken reports null.
CSRC = os.path.join(ROOT, "hyper_connection_rank_amd", "csrc")
_DEC_SRC = ("hc_decode.hip", "hc_device.h", "hc_mfma_common.h", "hc_internal.h")
_PF_SRC = ("hc_prefill.hip", "hc_decode.hip", "hc_device.h", "hc_mfma_common.h", "hc_internal.h")
TRAFFIC_SOURCES = {"hc_down": _DEC_SRC, "hc_uppre": _DEC_SRC, "pf_rms": _PF_SRC, "pf_down": _PF_SRC,
                   "inv_rms": ("hc_invrms.hip", "hc_device.h", "hc_internal.h"),
                   "pf_up2": _PF_SRC}
_DEC_PROFILE, _PF_PROFILE = "decode_block_rows1_bf16.md", "prefill_block_rows8192_bf16.md"
TRAFFIC_PROFILES = {"hc_down": _DEC_PROFILE, "hc_uppre": _DEC_PROFILE, "pf_rms": _PF_PROFILE,
                    "inv_rms": "inv_rms_rows8192_dim16384_bf16.md",
                    "pf_down": _PF_PROFILE, "pf_up2": _PF_PROFILE}


def sources_sha256(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from the
    kernel's committed counter summary, or None when there is none or the
    kernel's sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_PROFILES.get(kernel, ""))
    if kernel not in TRAFFIC_PROFILES or not os.path.isfile(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic_record:"):
                r = dict(kv.split("=", 1) for kv in line.split(":", 1)[1].split())
                if r.get("kernel") == kernel:
                    rec = r
    if rec.get("sources_sha256") != sources_sha256(kernel):
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()  # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    return evs


def sleep_cycles_per_ms():
    """Calibrate torch.cuda._sleep so the host can queue work ahead of the GPU."""
    import torch
    a, b = make_events(2)
    a.record()
    torch.cuda._sleep(1_000_000)
    b.record()
    torch.cuda.synchronize()
    return 1_000_000 / max(a.elapsed_time(b), 1e-3)


def per_kernel_times(calls, reps, kernels):
    """Average duration of each kernel (us) over `reps` passes of `calls`, each
    call an hclrmix_run_timed closure taking a list of events. Every kernel is
    dispatched with its own start/stop event pair (hipExtLaunchKernel), so the
    interval is that dispatch's execution time on the stream it runs on. The
    GPU is held by a sleep kernel while the host queues the work, so kernels
    run back to back as they do in the timed graph replay."""
    import torch
    per_call = 2 * kernels
    total = len(calls) * reps
    evs = make_events(per_call * total)
    pad = make_events(2 * MAX_KERNELS - per_call) if per_call < 2 * MAX_KERNELS else []
    cyc = sleep_cycles_per_ms()
    torch.cuda._sleep(int(cyc * min(200.0, 0.05 * total + 20)))
    i = 0
    for _ in range(reps):
        for call in calls:
            k = call(evs[i * per_call:(i + 1) * per_call] + pad)
            assert k == kernels, (k, kernels)
            i += 1
    torch.cuda.synchronize()
    sums = [0.0] * kernels
    for j in range(total):
        for k in range(kernels):
            sums[k] += evs[j * per_call + 2 * k].elapsed_time(evs[j * per_call + 2 * k + 1]) * 1000.0
    return [s / total for s in sums]


def timed_chain_calls(hc, weights, sets, ws, prob, attrs):
    """One hclrmix_run_chained closure per block of the chain (block b reads
    sets[b % 2] and writes sets[(b + 1) % 2]), taking the events to stamp."""
    nb = len(weights)
    calls = []
    for b in range(nb):
        i, o = sets[b % 2], sets[(b + 1) % 2]
        W, N = weights[b], weights[(b + 1) % nb]
        calls.append(lambda evs, i=i, o=o, W=W, N=N: hc.hclrmix_run_chained(
            i["streams"], W["norm_scale"], W["down_weight"], W["up_weight"], W["inject_weight"],
            i["pre"], i["post"], o["pre"], o["post"], o["streams"], ws, prob, attrs,
            next_down_weight=N["down_weight"], next_inject_weight=N["inject_weight"],
            events=[e.cuda_event for e in evs]))
    return calls


def bench_decode(args, hc, synth, torch):
    w = synth.WORKLOADS["decode_bf16"]
    nb = args.blocks
    t0 = time.time()
    weights = []
    for b in range(nb):
        t = synth.block_inputs(w, b, with_acts=False)
        weights.append({k: v.cuda() for k, v in t.items()})
    acts0 = {k: v.cuda() for k, v in synth.block_inputs(w, 0, with_weights=False).items()}
    log(f"decode: {nb} weight sets generated and copied in {time.time() - t0:.1f}s")
    dt = torch.bfloat16
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(1, w.K, w.R, hc.HCLRMIX_BF16, True)
    assert hc.hclrmix_select_path(prob, attrs) == hc.PATH_DECODE
    ws = hc.new_workspace(prob, attrs, "cuda")
    sets = [dict(streams=torch.empty(1, w.K, dtype=dt, device="cuda"),
                 pre=torch.empty(1, w.H, dtype=dt, device="cuda"),
                 post=torch.empty(1, w.C, dtype=dt, device="cuda")) for _ in range(2)]

    def reset():
        sets[0]["streams"].copy_(acts0["streams"])
        sets[0]["pre"].copy_(acts0["prev_block_output"])
        sets[0]["post"].copy_(acts0["prev_post_gate"])

    # A chain as a model runs it: each call is given the next block's down
    # and inject weights (hclrmix_run_chained), which it brings into cache
    # while it runs; `chained=False` is the plain hclrmix_run chain.
    def chain(n, chained=True):
        for b in range(n):
            i, o = sets[b % 2], sets[(b + 1) % 2]
            W, N = weights[b], weights[(b + 1) % nb]
            if chained:
                hc.hclrmix_run_chained(i["streams"], W["norm_scale"], W["down_weight"], W["up_weight"],
                                       W["inject_weight"], i["pre"], i["post"], o["pre"], o["post"],
                                       o["streams"], ws, prob, attrs, next_down_weight=N["down_weight"],
                                       next_inject_weight=N["inject_weight"])
            else:
                hc.hclrmix_run(i["streams"], W["norm_scale"], W["down_weight"], W["up_weight"],
                               W["inject_weight"], i["pre"], i["post"], o["pre"], o["post"], o["streams"],
                               ws, prob, attrs)

    reset()
    chain(nb)
    torch.cuda.synchronize()
    graphs = {}
    for n, chained in sorted({(nb, True), (nb // 2, True), (nb, False)}):
        reset()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            chain(n, chained)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            chain(n, chained)
        graphs[n if chained else -n] = g
    torch.cuda.synchronize()
    log("decode: graphs captured")

    # Timed region: exactly `steps` replays of the nb-block graph.
    reset()
    for _ in range(args.warmup):
        graphs[nb].replay()
    torch.cuda.synchronize()
    e0, e1 = make_events(2)
    e0.record()
    for _ in range(args.steps):
        graphs[nb].replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    us_block = ms_step * 1000.0 / nb
    log(f"decode: {ms_step:.3f} ms per {nb}-block replay = {us_block:.3f} us/block")

    # The pages' slope: (t_nb - t_nb/2) / (nb/2), min over repeats.
    def best(g, reps, inner):
        vals = []
        for _ in range(reps):
            a, b = make_events(2)
            a.record()
            for _ in range(inner):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            vals.append(a.elapsed_time(b) / inner)
        return min(vals)

    half = nb // 2
    t_full, t_half = best(graphs[nb], 5, 20), best(graphs[half], 5, 20)
    slope = (t_full - t_half) * 1000.0 / (nb - half)
    log(f"decode: slope {slope:.3f} us/block (t{nb}={t_full:.3f} ms, t{half}={t_half:.3f} ms)")
    reset()
    us_plain = best(graphs[-nb], 3, 20) * 1000.0 / nb
    log(f"decode: {us_plain:.3f} us/block with plain hclrmix_run calls (no next-block prefetch)")

    # Per-kernel durations (HIP events between the kernels, same stream).
    reset()
    names = KERNELS[1]
    kt = per_kernel_times(timed_chain_calls(hc, weights, sets, ws, prob, attrs), 3, len(names))
    log("decode kernels: " + ", ".join(f"{n} {t:.2f} us" for n, t in zip(names, kt)))
    alg = {"hc_down": DEC_DOWN_BYTES + DEC_POST_BYTES, "hc_uppre": DEC_UP_BYTES}
    dom = max(range(len(names)), key=lambda k: kt[k])
    achieved = alg[names[dom]] / (kt[dom] * 1e-6) / 1e9
    roof = {"kernel": names[dom], "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": recorded_traffic(names[dom]),
            "algorithmic_bytes_per_launch": alg[names[dom]], "avg_launch_us": round(kt[dom], 3)}
    del weights, graphs
    torch.cuda.empty_cache()
    return dict(us_block=us_block, ms_step=ms_step, slope=slope, kernels=dict(zip(names, kt)), roofline=roof,
                t_full=t_full, t_half=t_half, us_plain=us_plain)


def bench_prefill(args, hc, synth, torch):
    w = synth.WORKLOADS["prefill_bf16"]
    t0 = time.time()
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    log(f"prefill: inputs generated and copied in {time.time() - t0:.1f}s")
    dt = torch.bfloat16
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(w.rows, w.K, w.R, hc.HCLRMIX_BF16, True)
    assert hc.hclrmix_select_path(prob, attrs) == hc.PATH_PREFILL
    ws = hc.new_workspace(prob, attrs, "cuda")
    pre = torch.empty(w.rows, w.H, dtype=dt, device="cuda")
    post = torch.empty(w.rows, w.C, dtype=dt, device="cuda")
    so = torch.empty(w.rows, w.K, dtype=dt, device="cuda")
    args_t = (t["streams"], t["norm_scale"], t["down_weight"], t["up_weight"], t["inject_weight"],
              t["prev_block_output"], t["prev_post_gate"], pre, post, so, ws, prob, attrs)
    for _ in range(3):
        hc.hclrmix_run(*args_t)
    torch.cuda.synchronize()
    # One call between two events also counts the host's validation and
    # enqueue before the first kernel starts; bursts of back-to-back calls
    # give the device time per block (the single-call median is kept beside).
    single = []
    for _ in range(max(5, args.prefill_iters)):
        a, b = make_events(2)
        a.record()
        hc.hclrmix_run(*args_t)
        b.record()
        torch.cuda.synchronize()
        single.append(a.elapsed_time(b))
    burst = 10
    times = []
    for _ in range(5):
        a, b = make_events(2)
        a.record()
        for _ in range(burst):
            hc.hclrmix_run(*args_t)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / burst)
    ms = statistics.median(times)
    names = KERNELS[2]
    kt = per_kernel_times([lambda evs: hc.hclrmix_run_timed(*args_t, [e.cuda_event for e in evs])], 5, len(names))
    tflops = PF_FLOP / (ms * 1e-3) / 1e12
    log(f"prefill: {ms * 1000:.1f} us per block in bursts of {burst} ({statistics.median(single) * 1000:.1f} us "
        f"for one call alone), {tflops:.1f} TFLOP/s; kernels "
        + ", ".join(f"{n} {x:.1f} us" for n, x in zip(names, kt)))
    flop_k = {"pf_rms": 0, "pf_down": 2 * w.rows * w.K * (w.R + w.C), "reduce_prep": 0,
              "pf_up2": 2 * w.rows * w.R * w.K}
    dom = max((k for k in range(len(names)) if flop_k[names[k]]), key=lambda k: kt[k])
    ach = flop_k[names[dom]] / (kt[dom] * 1e-6) / 1e12
    roof = {"kernel": names[dom], "bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": recorded_traffic(names[dom]),
            "algorithmic_flop_per_launch": flop_k[names[dom]], "avg_launch_us": round(kt[dom], 2)}
    torch.cuda.synchronize()
    outs = (pre.cpu(), post.cpu(), so.cpu())
    return dict(us=ms * 1000, us_single=statistics.median(single) * 1000, burst=burst, tflops=tflops,
                kernels=dict(zip(names, kt)), roofline=roof, outputs=outs)


def chain_slope(hc, synth, torch, w, nsets: int, n_hi: int, n_lo: int, chained: bool):
    """µs/block of a chain of blocks of workload `w` over `nsets` distinct
    seeded weight sets (block b takes set b mod nsets; each block's streams,
    and with a prologue its prev_out and prev_gate, are the previous block's
    outputs), as the slope (t_hi - t_lo) / (n_hi - n_lo) between HIP graphs
    of n_hi and n_lo blocks, the min over repeats."""
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    code = {"bf16": hc.HCLRMIX_BF16, "f16": hc.HCLRMIX_F16, "f32": hc.HCLRMIX_F32}[w.dtype]
    weights = [{k: v.cuda() for k, v in synth.block_inputs(w, b, with_acts=False).items()} for b in range(nsets)]
    acts0 = {k: v.cuda() for k, v in synth.block_inputs(w, 0, with_weights=False).items()}
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(w.rows, w.K, w.R, code, w.has_prologue)
    ws = hc.new_workspace(prob, attrs, "cuda")
    sets = [dict(streams=torch.empty(w.rows, w.K, dtype=dt, device="cuda"),
                 pre=torch.empty(w.rows, w.H, dtype=dt, device="cuda"),
                 post=torch.empty(w.rows, w.C, dtype=dt, device="cuda")) for _ in range(2)]
    sets[0]["streams"].copy_(acts0["streams"])
    if w.has_prologue:
        sets[0]["pre"].copy_(acts0["prev_block_output"])
        sets[0]["post"].copy_(acts0["prev_post_gate"])

    def chain(n):
        for b in range(n):
            i, o = sets[b % 2], sets[(b + 1) % 2]
            W, N = weights[b % nsets], weights[(b + 1) % nsets]
            po, pg = (i["pre"], i["post"]) if w.has_prologue else (None, None)
            if chained:
                hc.hclrmix_run_chained(i["streams"], W["norm_scale"], W["down_weight"], W["up_weight"],
                                       W["inject_weight"], po, pg, o["pre"], o["post"], o["streams"], ws, prob,
                                       attrs, next_down_weight=N["down_weight"],
                                       next_inject_weight=N["inject_weight"])
            else:
                hc.hclrmix_run(i["streams"], W["norm_scale"], W["down_weight"], W["up_weight"], W["inject_weight"],
                               po, pg, o["pre"], o["post"], o["streams"], ws, prob, attrs)

    chain(2)
    torch.cuda.synchronize()
    graphs = {}
    for n in (n_hi, n_lo):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            chain(n)
        torch.cuda.current_stream().wait_stream(st)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            chain(n)
        graphs[n] = g
    torch.cuda.synchronize()
    t = {}
    for n, g in graphs.items():
        g.replay()
        torch.cuda.synchronize()
        vals = []
        for _ in range(5):
            a, b = make_events(2)
            a.record()
            for _ in range(5):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            vals.append(a.elapsed_time(b) / 5)
        t[n] = min(vals)
    us = (t[n_hi] - t[n_lo]) * 1000.0 / (n_hi - n_lo)
    del weights, graphs, sets, ws
    torch.cuda.empty_cache()
    return us


def bench_other_configs(hc, synth, torch):
    """The remaining workloads, reported beside the bench line: the tiny fp32
    block (median of 100 single calls, each between two events, so host time
    counts), the rows=8 decode chain (96 distinct weight sets, 96 vs 48 block
    graphs) and the wide fp16 block (16 distinct weight sets of 67.7 MB, more
    than the memory-side cache, 16 vs 8 block graphs)."""
    out = {}
    w = synth.WORKLOADS["tiny_f32"]
    t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(w.rows, w.K, w.R, hc.HCLRMIX_F32, True)
    ws = hc.new_workspace(prob, attrs, "cuda")
    o = (torch.empty(w.rows, w.H, device="cuda"), torch.empty(w.rows, w.C, device="cuda"),
         torch.empty(w.rows, w.K, device="cuda"))
    args_t = (t["streams"], t["norm_scale"], t["down_weight"], t["up_weight"], t["inject_weight"],
              t["prev_block_output"], t["prev_post_gate"], *o, ws, prob, attrs)
    for _ in range(5):
        hc.hclrmix_run(*args_t)
    torch.cuda.synchronize()
    vals = []
    for _ in range(100):
        a, b = make_events(2)
        a.record()
        hc.hclrmix_run(*args_t)
        b.record()
        torch.cuda.synchronize()
        vals.append(a.elapsed_time(b) * 1000.0)
    out["tiny_f32"] = {"workload": w.name, "path": "generic", "us_per_call": round(statistics.median(vals), 2),
                       "timing": "median of 100 single calls between two events (host time included)"}
    w = synth.WORKLOADS["decode_chain_bf16"]
    us = chain_slope(hc, synth, torch, w, 96, 96, 48, True)
    nbytes = 13209600 + w.rows * (2 * w.K * 2 + w.H * 2 * 2 + w.C * 2 * 2)  # weights + activations
    out["decode_chain_bf16"] = {"workload": w.name, "path": "decode", "us_per_block": round(us, 3),
                                "hbm_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                                "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                                "timing": "slope of 96- and 48-block graphs of chained calls"}
    w = synth.WORKLOADS["wide_f16"]
    us = chain_slope(hc, synth, torch, w, 16, 16, 8, False)
    nbytes = (w.K * w.R * 2 * 2 + w.K * w.C * 2 + w.K * 2) + w.rows * (2 * w.K * 2 + w.H * 2 + w.C * 2)
    out["wide_f16"] = {"workload": w.name, "path": "decode" if w.rows <= 16 else "prefill",
                       "us_per_block": round(us, 2), "hbm_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                       "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                       "timing": "slope of 16- and 8-block graphs over 16 distinct weight sets"}
    for k, v in out.items():
        log(f"{k}: " + ", ".join(f"{a} {b}" for a, b in v.items() if a not in ("workload", "timing")))
    return out


def cpu_baseline(synth, seconds: float, hc=None, torch=None):
    """The oracle as it stands, on the same decode workload, one block (rows = 1)
    at a time until `seconds` of CPU work; a row uses one thread. Its outputs
    are then set against the GPU's for the same inputs (one hclrmix_run)."""
    import oracle
    w = synth.WORKLOADS["decode_bf16"]
    t = synth.block_inputs(w)
    args = [t[n] for n in ("streams", "norm_scale", "down_weight", "up_weight", "inject_weight",
                           "prev_block_output", "prev_post_gate")]
    n, t0 = 0, time.time()
    while time.time() - t0 < seconds or n < 2:
        ora = oracle.run(*args, **w.attrs(), threads=1, want_mag=True)
        n += 1
    el = time.time() - t0
    res = {"value": round(el / n * 1e6, 1), "unit": "us/block", "cores": 1, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n} decode blocks (rows=1, 4x2560, R=320, bf16) in {el:.1f}s, one thread "
                     f"(one row gives the oracle one thread of work)"}
    if hc is not None:
        gpu = hc.block(*[None if a is None else a.cuda() for a in args], **w.attrs())
        torch.cuda.synchronize()
        res["agreement"] = agreement([x.cpu() for x in gpu], ora[:3], ora[3])
    return res


def cpu_prefill_sample(synth, rows: int, gpu_out=None):
    """The oracle on `rows` rows of the prefill workload, all host threads it
    may use; with the GPU's outputs of the full block, their agreement."""
    import oracle
    w = synth.WORKLOADS["prefill_bf16"]
    t = synth.block_inputs(w, rows=rows)
    args = [t[n] for n in ("streams", "norm_scale", "down_weight", "up_weight", "inject_weight",
                           "prev_block_output", "prev_post_gate")]
    th = oracle.default_threads()
    t0 = time.time()
    ora = oracle.run(*args, **w.attrs(), threads=th, want_mag=True)
    el = time.time() - t0
    flop = 2 * rows * w.K * (2 * w.R + w.C)
    res = {"tflops": round(flop / el / 1e12, 4), "cores": th, "cpu_model": cpu_model(),
           "sample": f"{rows} of {w.rows} prefill rows in {el:.2f}s"}
    if gpu_out is not None:
        res["agreement"] = agreement([g[:rows] for g in gpu_out], ora[:3], ora[3])
    return res


def trace_pass(args, hc, synth, torch):
    """Only the timed configuration, for a kernel-trace run (rocprofv3
    --kernel-trace --stats): the graph of `blocks` chained decode calls over
    distinct weight sets that the bench line times, replayed warmup + steps
    times. Besides it, the only dispatches are one eager chained call (the
    first two kernels of the run, before the capture) and the input copies."""
    w = synth.WORKLOADS["decode_bf16"]
    nb = args.blocks
    weights = [{k: v.cuda() for k, v in synth.block_inputs(w, b, with_acts=False).items()} for b in range(nb)]
    acts0 = {k: v.cuda() for k, v in synth.block_inputs(w, 0, with_weights=False).items()}
    dt = torch.bfloat16
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(1, w.K, w.R, hc.HCLRMIX_BF16, True)
    ws = hc.new_workspace(prob, attrs, "cuda")
    sets = [dict(streams=acts0["streams"].clone(), pre=acts0["prev_block_output"].clone(),
                 post=acts0["prev_post_gate"].clone()),
            dict(streams=torch.empty(1, w.K, dtype=dt, device="cuda"), pre=torch.empty(1, w.H, dtype=dt, device="cuda"),
                 post=torch.empty(1, w.C, dtype=dt, device="cuda"))]

    def call(b):
        i, o = sets[b % 2], sets[(b + 1) % 2]
        W, N = weights[b], weights[(b + 1) % nb]
        hc.hclrmix_run_chained(i["streams"], W["norm_scale"], W["down_weight"], W["up_weight"], W["inject_weight"],
                               i["pre"], i["post"], o["pre"], o["post"], o["streams"], ws, prob, attrs,
                               next_down_weight=N["down_weight"], next_inject_weight=N["inject_weight"])

    call(0)
    torch.cuda.synchronize()
    if args.trace_eager:
        # the dispatches bench.py's per-kernel event timing measures (the
        # source of the line's roofline): the same chained calls, back to back
        kt = per_kernel_times(timed_chain_calls(hc, weights, sets, ws, prob, attrs), 3, 2)
        log(f"trace pass: {3 * nb} event-timed chained calls; events: "
            + ", ".join(f"{n} {t:.3f} us" for n, t in zip(KERNELS[1], kt)))
        return
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for b in range(nb):
            call(b)
    for _ in range(args.warmup + args.steps):
        g.replay()
    torch.cuda.synchronize()
    log(f"trace pass: {args.warmup + args.steps} replays of the {nb}-block chained graph done")


def profile_pass(args, hc, synth, torch):
    """Untimed eager work for hardware-counter runs (rocprofv3 --pmc): the
    decode chain of chained calls over `blocks` distinct weight sets, the rows = 8192 prefill
    block three times, and a plain device copy of COPY_BYTES three times; the
    copy's counters per byte calibrate the block kernels' counters."""
    w = synth.WORKLOADS["decode_bf16"]
    dt = torch.bfloat16
    attrs = hc.make_attrs(**w.attrs())
    prob = hc.make_problem(1, w.K, w.R, hc.HCLRMIX_BF16, True)
    ws = hc.new_workspace(prob, attrs, "cuda")
    a0 = {k: v.cuda() for k, v in synth.block_inputs(w, 0, with_weights=False).items()}
    io = [dict(s=a0["streams"].clone(), p=a0["prev_block_output"].clone(), g=a0["prev_post_gate"].clone()),
          dict(s=torch.empty(1, w.K, dtype=dt, device="cuda"), p=torch.empty(1, w.H, dtype=dt, device="cuda"),
               g=torch.empty(1, w.C, dtype=dt, device="cuda"))]
    Ws = [{k: v.cuda() for k, v in synth.block_inputs(w, b, with_acts=False).items()} for b in range(args.blocks)]
    for b in range(args.blocks):  # chained calls, as the bench line times them
        W, N = Ws[b], Ws[(b + 1) % args.blocks]
        i, o = io[b % 2], io[(b + 1) % 2]
        hc.hclrmix_run_chained(i["s"], W["norm_scale"], W["down_weight"], W["up_weight"], W["inject_weight"],
                               i["p"], i["g"], o["p"], o["g"], o["s"], ws, prob, attrs,
                               next_down_weight=N["down_weight"], next_inject_weight=N["inject_weight"])
    torch.cuda.synchronize()
    del Ws
    log(f"profile pass: {args.blocks} chained decode blocks done")
    if not args.no_prefill:
        w = synth.WORKLOADS["prefill_bf16"]
        t = {k: v.cuda() for k, v in synth.block_inputs(w).items()}
        attrs = hc.make_attrs(**w.attrs())
        prob = hc.make_problem(w.rows, w.K, w.R, hc.HCLRMIX_BF16, True)
        ws = hc.new_workspace(prob, attrs, "cuda")
        pre = torch.empty(w.rows, w.H, dtype=dt, device="cuda")
        post = torch.empty(w.rows, w.C, dtype=dt, device="cuda")
        so = torch.empty(w.rows, w.K, dtype=dt, device="cuda")
        for _ in range(3):
            hc.hclrmix_run(t["streams"], t["norm_scale"], t["down_weight"], t["up_weight"], t["inject_weight"],
                           t["prev_block_output"], t["prev_post_gate"], pre, post, so, ws, prob, attrs)
        torch.cuda.synchronize()
        log("profile pass: 3 prefill blocks done")
    if not args.no_prefill:
        x = torch.randn(IR_ROWS, IR_DIM, device="cuda").to(dt)
        for _ in range(3):
            hc.hclrmix_inv_rms(x, 1e-6)
        torch.cuda.synchronize()
        del x
        log("profile pass: 3 inv_rms calls done")
    src = torch.ones(COPY_BYTES // 2, dtype=dt, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"profile pass: 3 copies of {COPY_BYTES} bytes done")


COPY_BYTES = 256 << 20  # calibration copy: reads and writes this many bytes


IR_ROWS, IR_DIM = 8192, 16384  # the pre-norm page's full size (hc_dim 16384)


def bench_inv_rms(args, hc, torch):
    """Standalone inv_rms at the pre-norm page's size: 8192 bf16 rows of
    16384; one value per row. Bytes per call: the source once plus the fp32
    results. The source is rotated over copies that exceed the memory-side
    cache, so each call reads HBM."""
    import math
    copies = max(2, math.ceil(2 * 256 * 2**20 / (IR_ROWS * IR_DIM * 2)) + 1)
    g = torch.Generator(device="cuda").manual_seed(77)
    xs = [torch.randn(IR_ROWS, IR_DIM, device="cuda", generator=g).to(torch.bfloat16) for _ in range(copies)]
    out = torch.empty(IR_ROWS, dtype=torch.float32, device="cuda")
    for x in xs:
        hc.hclrmix_inv_rms(x, 1e-6, out=out)
    torch.cuda.synchronize()
    reps = 10 * copies
    a, b = make_events(2)
    a.record()
    for i in range(reps):
        hc.hclrmix_inv_rms(xs[i % copies], 1e-6, out=out)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / reps
    nbytes = IR_ROWS * IR_DIM * 2 + IR_ROWS * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    log(f"inv_rms: {us:.1f} us per call ({IR_ROWS} x {IR_DIM} bf16), {gbps:.0f} GB/s")
    del xs
    torch.cuda.empty_cache()
    return dict(us=us, gbps=gbps, nbytes=nbytes)


def measure_peaks(torch):
    """Achievable peaks of this GPU, from libhcpeaks: HBM read and copy over
    1 GiB buffers (four times the 256 MB memory-side cache; non-temporal
    16-byte accesses) and dense bf16 matrix-core throughput (16x16x32:
    sixteen independent chains per wave, 32 waves per compute unit; 32x32x16:
    four chains, sixteen waves; the occupancy each runs fastest at)."""
    import ctypes
    from hyper_connection_rank_amd import build as B
    if not os.path.exists(B.PEAKS_LIB):
        raise RuntimeError(f"{B.PEAKS_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(B.PEAKS_LIB)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.hcpeaks_read.argtypes = [vp, sz, vp, vp]
    lib.hcpeaks_copy.argtypes = [vp, vp, sz, vp]
    lib.hcpeaks_mfma_bf16.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    for f in (lib.hcpeaks_read, lib.hcpeaks_copy, lib.hcpeaks_mfma_bf16):
        f.restype = ctypes.c_int
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, big_blocks, iters = 8 * cus, 4 * cus, 4096  # the occupancy each instruction runs fastest at
    fsink = torch.empty(4 * blocks, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(call, reps):
        for _ in range(2):
            if call() != 0:
                raise RuntimeError("libhcpeaks launch failed")
        a, b = make_events(2)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps  # seconds per call

    t_read = timed(lambda: lib.hcpeaks_read(src.data_ptr(), n, sink.data_ptr(), stream), 20)
    t_copy = timed(lambda: lib.hcpeaks_copy(src.data_ptr(), dst.data_ptr(), n, stream), 20)
    t_small = timed(lambda: lib.hcpeaks_mfma_bf16(fsink.data_ptr(), blocks, iters, 0, stream), 5)
    t_big = timed(lambda: lib.hcpeaks_mfma_bf16(fsink.data_ptr(), big_blocks, iters, 1, stream), 5)
    flop_small = 4 * 16 * iters * 16384  # per workgroup: 4 waves x 16 chains of 16x16x32
    flop_big = 4 * 4 * iters * 32768     # per workgroup: 4 waves x 4 chains of 32x32x16
    peaks = {"hbm_read_gbps": round(n / t_read / 1e9, 1), "hbm_copy_gbps": round(2 * n / t_copy / 1e9, 1),
             "mfma_bf16_tflops": round(blocks * flop_small / t_small / 1e12, 1),
             "mfma_bf16_32x32x16_tflops": round(big_blocks * flop_big / t_big / 1e12, 1),
             "method": "libhcpeaks: 1 GiB non-temporal read / copy, 32 KB per workgroup (copy counts both "
                       f"directions); {blocks} (16x16x32) or {big_blocks} (32x32x16) workgroups x 4 waves of "
                       "bf16 matrix ops on register operands, "
                       "mfma_bf16_tflops with 16x16x32 (the instruction of the fixed summation order), "
                       "mfma_bf16_32x32x16_tflops with 32x32x16"}
    del src, dst, sink, fsink
    torch.cuda.empty_cache()
    log(f"measured peaks: read {peaks['hbm_read_gbps']} GB/s, copy {peaks['hbm_copy_gbps']} GB/s, "
        f"bf16 matrix {peaks['mfma_bf16_tflops']} TFLOP/s (16x16x32), "
        f"{peaks['mfma_bf16_32x32x16_tflops']} TFLOP/s (32x32x16)")
    return peaks


def _peaks_lib():
    import ctypes
    from hyper_connection_rank_amd import build as B
    if not os.path.exists(B.PEAKS_LIB):
        raise RuntimeError(f"{B.PEAKS_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(B.PEAKS_LIB)
    vp, sz, ci, cu = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint
    lib.hcpeaks_empty.argtypes = [ci, vp]
    lib.hcpeaks_stream.argtypes = [vp, sz, ci, ci, vp, vp, cu, vp, vp]
    for f in (lib.hcpeaks_empty, lib.hcpeaks_stream):
        f.restype = ctypes.c_int
    return lib


def measure_overlap(torch, steps: int = 2000):
    """Cycles per step per SIMD (2.4 GHz) of libhcpeaks' overlap probe: two
    waves per SIMD, a step being 16 independent 16x16x32 bf16 matrix ops
    and/or 64 independent fp32 vector ops per wave; the four modes put both
    kinds in separate runs, interleaved in every wave, or in different waves."""
    lib = _peaks_lib()
    import ctypes
    lib.hcpeaks_overlap.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hcpeaks_overlap.restype = ctypes.c_int
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * blocks, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    names = ("matrix_only", "vector_only", "both_interleaved_in_each_wave", "one_wave_of_each_kind")
    out = {}
    for mode, name in enumerate(names):
        best = None
        for _ in range(5):
            a, b = make_events(2)
            a.record()
            if lib.hcpeaks_overlap(sink.data_ptr(), blocks, steps, mode, stream) != 0:
                raise RuntimeError("libhcpeaks overlap launch failed")
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None else min(best, t)
        out[name] = round(best * 2.4e9 / (2 * steps), 1)
    out["unit"] = "cycles per step per SIMD at 2.4 GHz (best of 5)"
    out["step"] = "16 matrix ops 16x16x32 bf16 and/or 64 fp32 vector ops per wave, two waves per SIMD"
    return out


def measure_floors(torch, nb: int = 96):
    """Floors of one decode block on this GPU, as µs per launch in HIP graphs
    of `nb` launches (the slope between graphs of nb and nb/2 launches, the
    min over repeats, as the decode chain is timed): an empty kernel of 256
    workgroups; one kernel streaming 6,553,600 bytes (one weight matrix of the
    block) and one streaming 13,209,600 bytes (all of its weights), each
    launch on a different buffer (1.27 GB in all, more than the memory-side
    cache); a grid barrier of 256 workgroups alone; and the 13.2 MB stream
    followed by that barrier (the least a one-kernel block does)."""
    lib = _peaks_lib()
    stream = torch.cuda.current_stream().cuda_stream
    full, half_w = 13209600, 6553600
    bufs = [torch.full((full // 4,), b + 1, dtype=torch.int32, device="cuda") for b in range(nb)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sync = torch.zeros(128, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    spin = 1 << 20
    G = 256

    def graph_of(n, call):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for i in range(n):
                assert call(i, torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.current_stream().wait_stream(st)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                assert call(i, torch.cuda.current_stream().cuda_stream) == 0
        return g

    def per_launch(call):
        gs = {n: graph_of(n, call) for n in (nb, nb // 2)}
        t = {}
        for n, g in gs.items():
            g.replay()
            torch.cuda.synchronize()
            vals = []
            for _ in range(5):
                a, b = make_events(2)
                a.record()
                for _ in range(5):
                    g.replay()
                b.record()
                torch.cuda.synchronize()
                vals.append(a.elapsed_time(b) / 5)
            t[n] = min(vals)
        return round((t[nb] - t[nb // 2]) * 1000.0 / (nb - nb // 2), 3), round(t[nb] * 1000.0 / nb, 3)

    def stream_call(nbytes, barrier):
        return lambda i, st: lib.hcpeaks_stream(bufs[i % nb].data_ptr() if nbytes else None, nbytes, G, barrier,
                                                sink.data_ptr(), sync.data_ptr(), spin, err.data_ptr(), st)

    out = {}
    for key, call in (("empty_kernel", lambda i, st: lib.hcpeaks_empty(G, st)),
                      ("stream_6.55MB", stream_call(half_w, 0)),
                      ("stream_13.2MB", stream_call(full, 0)),
                      ("grid_barrier", stream_call(0, 1)),
                      ("stream_13.2MB_then_barrier", stream_call(full, 1))):
        slope, mean = per_launch(call)
        out[key] = {"us_per_launch_slope": slope, "us_per_launch_mean": mean}
    torch.cuda.synchronize()
    out["barrier_spin_timeouts"] = int(err.item())
    out["method"] = (f"libhcpeaks kernels of {G} workgroups x 256 threads in HIP graphs of {nb} and {nb // 2} "
                     "launches; slope = (t_nb - t_nb/2) / (nb/2), min of 5 x 5 replays; streams read a different "
                     f"buffer each launch ({nb} buffers of 13.2 MB); barrier = self-resetting arrival counter "
                     "and generation word, relaxed agent-scope atomics, bounded spin")
    del bufs
    torch.cuda.empty_cache()
    log("floors: " + ", ".join(f"{k} {v['us_per_launch_slope']} us" for k, v in out.items() if isinstance(v, dict)))
    return out


def _ordered16(x):
    """16-bit floats as integers ordered like their values (+0 == -0)."""
    b = x.contiguous().view(torch_mod().int16).to(torch_mod().int64) & 0xFFFF
    return torch_mod().where(b >= 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def torch_mod():
    import torch
    return torch


def agreement(gpu, ora, mag=None):
    """GPU outputs against the oracle's on the same inputs: bit-exact share,
    largest distance in ulps of T, and how many elements more than 2 ulps
    apart are within 2 ulps of the magnitude feeding their last rounding
    (cancellation; `mag` = |rs| * sum_c |hn * g| for pre_output)."""
    torch = torch_mod()
    out = {}
    for name, g, o in zip(("pre_output", "post_gate", "streams_out"), gpu, ora):
        d = (_ordered16(g) - _ordered16(o)).abs()
        far = d > 2
        rej = 0
        if name == "pre_output" and mag is not None and bool(far.any()):
            m = mag.double().abs()
            ulp = torch.pow(2.0, torch.floor(torch.log2(torch.clamp(m, min=2.0 ** -126))) - 7)
            rej = int((far & ((g.double() - o.double()).abs() <= 2 * ulp)).sum())
        out[name] = {"n": int(d.numel()), "exact_frac": round(float((d == 0).double().mean()), 6),
                     "max_ulp": int(d.max()), "rejudged": rej, "beyond_tolerance": int(far.sum()) - rej}
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_inv_rms_sample(torch, rows: int, seconds: float = 2.0):
    """The oracle's inv_rms on `rows` rows of the same size (one thread),
    repeated until `seconds` of CPU work."""
    import oracle
    x = torch.randn(rows, IR_DIM).to(torch.bfloat16)
    n, t0 = 0, time.time()
    while True:
        oracle.inv_rms(x, 1e-6)
        n += 1
        dt = time.time() - t0
        if dt >= seconds:
            break
    return {"value": round(n * rows * IR_DIM * 2 / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} passes over {rows} of {IR_ROWS} rows in {dt:.2f}s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed replays of the 96-block chain")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--blocks", type=int, default=96)
    ap.add_argument("--prefill-iters", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="untimed eager pass for hardware-counter runs; prints no JSON line")
    ap.add_argument("--trace-pass", action="store_true",
                    help="only the timed graph of chained decode calls, replayed warmup + steps times, for a "
                         "kernel-trace run; prints no JSON line")
    ap.add_argument("--trace-eager", action="store_true",
                    help="with --trace-pass: the event-timed chained calls the roofline comes from, not the graph")
    ap.add_argument("--probes", action="store_true",
                    help="only the matrix/vector overlap probe of libhcpeaks, as one JSON line")
    ap.add_argument("--others-pass", action="store_true",
                    help="only the timing runs of the three other configurations (tiny fp32 block, rows=8 "
                         "decode chain, wide fp16 block), for a kernel-trace run; logs their figures, no JSON line")
    ap.add_argument("--floors", action="store_true",
                    help="only the decode floors (empty kernel, cold weight streams, grid barrier); one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this block runs on one GPU; --gpus {args.gpus} is not supported "
              f"(rows shard across GPUs without communication, so per-GPU figures are the ones measured)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import hyper_connection_rank_amd as hc
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    log(f"device {torch.cuda.get_device_name(0)} ({torch.cuda.get_device_properties(0).gcnArchName})")
    if args.profile_pass:
        profile_pass(args, hc, synth, torch)
        return
    if args.trace_pass:
        trace_pass(args, hc, synth, torch)
        return
    if args.others_pass:
        bench_other_configs(hc, synth, torch)
        return
    if args.floors:
        print(json.dumps({"decode_floors": measure_floors(torch, args.blocks)}), flush=True)
        return
    if args.probes:
        print(json.dumps({"matrix_vector_overlap": measure_overlap(torch)}), flush=True)
        return
    dec = bench_decode(args, hc, synth, torch)
    floors = measure_floors(torch, args.blocks)
    pf = None if args.no_prefill else bench_prefill(args, hc, synth, torch)
    ir = None if args.no_prefill else bench_inv_rms(args, hc, torch)
    peaks = measure_peaks(torch)
    others = None if args.no_prefill else bench_other_configs(hc, synth, torch)
    cpu = None if args.no_cpu else cpu_baseline(synth, args.cpu_seconds, hc, torch)
    if cpu:
        log(f"cpu oracle: {cpu['value']} us/block ({cpu['sample']})")
    cpu_pf = None if (args.no_cpu or args.no_prefill) else cpu_prefill_sample(synth, 8192, pf["outputs"])
    line = {
        "metric": METRIC,
        "value": round(dec["us_block"], 4),
        "unit": "us/block",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_step"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs; distinct weights per block)",
        "config": {"workload": f"decode block rows=1 bf16 C=4 H=2560 R=320 prologue; {args.blocks}-block chain, "
                               "distinct weights, graph replay",
                   "calls": "hclrmix_run_chained (each call given the next block's down/inject weights)",
                   "rows": 1, "num_branches": 4, "hidden": 2560, "rank": 320, "blocks_per_step": args.blocks},
        "us_per_block_plain_calls": round(dec["us_plain"], 4),
        "hbm_gbps": round(DEC_BLOCK_BYTES / (dec["us_block"] * 1e-6) / 1e9, 1),
        "hbm_frac": round(DEC_BLOCK_BYTES / (dec["us_block"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "slope_us_per_block": round(dec["slope"], 4),
        "kernels_us": {k: round(v, 3) for k, v in dec["kernels"].items()},
        "roofline": dict(dec["roofline"], frac_of_measured_read_peak=round(
            dec["roofline"]["achieved"] / peaks["hbm_read_gbps"], 4)),
        "cpu_baseline": cpu,
        "measured_peaks": peaks,
        "decode_floors": floors,
    }
    if others:
        line["other_configs"] = others
    if cpu and "agreement" in cpu:
        line["agreement"] = {"decode_rows1": cpu["agreement"]}
        if cpu_pf and "agreement" in cpu_pf:
            line["agreement"]["prefill_rows8192"] = cpu_pf["agreement"]
        line["agreement"]["reference"] = ("the CPU oracle on the same inputs (bench's cpu_baseline leg); tolerance "
                                          "2 ulp of T, re-judged against 2 ulp of the summands' magnitude near "
                                          "cancellation")
    if pf:
        line["prefill"] = {"rows": PF_ROWS, "us": round(pf["us"], 1), "tflops": round(pf["tflops"], 2),
                           "timing": f"median of 5 bursts of {pf['burst']} back-to-back calls, per call",
                           "us_single_call": round(pf["us_single"], 1),
                           "mfma_frac": round(pf["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                           "hbm_gbps": round(PF_BYTES / (pf["us"] * 1e-6) / 1e9, 1),
                           "kernels_us": {k: round(v, 2) for k, v in pf["kernels"].items()},
                           # min(matrix peak, arithmetic intensity x HBM peak): the block's own roofline
                           "roofline_tflops": round(PF_ROOF_TFLOPS, 1),
                           "roofline_frac": round(pf["tflops"] / PF_ROOF_TFLOPS, 4),
                           "mfma_frac_of_measured": round(pf["tflops"] / peaks["mfma_bf16_tflops"], 4),
                           "roofline": dict(pf["roofline"], frac_of_measured_peak=round(
                               pf["roofline"]["achieved"] / peaks["mfma_bf16_tflops"], 4)),
                           "cpu_oracle": cpu_pf}
    if ir:
        line["inv_rms"] = {"rows": IR_ROWS, "dim": IR_DIM, "dtype": "bf16", "us": round(ir["us"], 2),
                           "bytes_per_call": ir["nbytes"], "hbm_gbps": round(ir["gbps"], 1),
                           "hbm_frac": round(ir["gbps"] / HBM_PEAK_GBPS, 4),
                           "frac_of_measured_read_peak": round(ir["gbps"] / peaks["hbm_read_gbps"], 4),
                           "traffic": recorded_traffic("inv_rms"),
                           "cpu_oracle": None if args.no_cpu else cpu_inv_rms_sample(torch, IR_ROWS)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
