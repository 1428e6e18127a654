"""CPU checks of the parity judge's last judgement for pre_output: the step
that pre_output = rT(rs * sum_c hn_c * g_c) takes when the rounded factors
hn_c and g_c each land one T step away from the oracle's (the pages' "Numerics
contract", onnxruntime PR #33384, rounds both once after sums whose order it
leaves open). Results built from the oracle's own traced factors, moved by one
step, must pass; a dropped branch or factors two steps away must not."""
from __future__ import annotations

import torch

import oracle
import synth
from _parity import NAMES, judge_block, oracle_run

ROWS, C, H, R = 6, 2, 40, 16


def _setup():
    w = synth.Workload(4242, "judge", ROWS, C, H, R, "bf16", True, epsilon=1e-6, reduction_scale=0.25,
                       silu_alpha=0.25, gate_div=4.0, gate_mul=2.0)
    t = synth.block_inputs(w)
    return w, t, oracle_run(t, w.attrs())


def _factors(t, attrs, r):
    one = {k: (v[r:r + 1].contiguous() if k in ("streams", "prev_block_output", "prev_post_gate") else v)
           for k, v in t.items()}
    tr = oracle.trace(*[one.get(n) for n in NAMES], row=0, **attrs)
    return tr["hn"].view(C, H), tr["g"].view(C, H)


def _steps(x: torch.Tensor, k: int) -> torch.Tensor:
    """x (fp32 holding bf16 values) moved k bf16 steps away from zero."""
    b = x.to(torch.bfloat16).view(torch.int16)
    return (b + k).view(torch.bfloat16).float()


def _pre(hn, g, rs, keep=None):
    acc = torch.zeros(H, dtype=torch.float32)
    for c in range(C):
        if keep is None or c in keep:
            acc = acc + hn[c] * g[c]
    return (rs * acc).to(torch.bfloat16)


def _judge_pre(w, t, o, make):
    rs = w.attrs()["reduction_scale"]
    pre = torch.stack([make(*_factors(t, w.attrs(), r), rs) for r in range(ROWS)])
    return judge_block((pre, o[1], o[2]), o, True)[0]


def test_one_step_in_each_factor_passes():
    # Both factors of every branch one step further from zero (or nearer):
    # the largest move the bound admits; some elements need the bound.
    w, t, o = _setup()
    for k in (1, -1):
        j = _judge_pre(w, t, o, lambda hn, g, rs: _pre(_steps(hn, k), _steps(g, k), rs))
        assert j.bad == 0 and j.extra.get("flip_judged", 0) > 0, j.summary()


def test_dropped_branch_fails():
    w, t, o = _setup()
    j = _judge_pre(w, t, o, lambda hn, g, rs: _pre(hn, g, rs, keep=(0,)))
    assert j.bad > ROWS * H // 2, j.summary()


def test_two_steps_in_each_factor_fail():
    w, t, o = _setup()
    for k in (2, -2):
        j = _judge_pre(w, t, o, lambda hn, g, rs: _pre(_steps(hn, k), _steps(g, k), rs))
        assert j.bad > ROWS * H // 2, j.summary()
