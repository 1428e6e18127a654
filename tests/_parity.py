"""Parity helpers: run a block on the GPU (through the C-ABI binding) and on
the CPU oracle with the same input bytes, and judge the outputs.

Tolerances (a row's GPU result against the oracle):
  fp32       |gpu - ora| <= 1e-5 * max(|ora|, mag)
  fp16/bf16  ulp distance in T <= 2; an element failing that is re-judged
             against |gpu - ora| <= 2 * ulp_T(mag) (cancellation in a sum);
             a pre_output element failing both is judged last against the
             step the pre-mix takes when its rounded factors hn_c and g_c
             each land one T step apart (below)
  streams_out is exact.
mag is the magnitude feeding the output's last rounding: |rs| * sum_c |hn*g|
for pre_output (from the oracle), |ora| otherwise.

The last judgement: the pages' "Numerics contract" (onnxruntime PR #33384)
rounds hn and g to T once each, but leaves the order of the sums before them
(the sum of squares, the down and up projections) to the implementation, so
two correct implementations may round any hn_c or g_c to adjacent T values.
pre_output = rT(rs * sum_c hn_c * g_c) then differs by at most
  |rs| * sum_c (ulp(hn_c) |g_c| + |hn_c| ulp(g_c) + ulp(hn_c) ulp(g_c)) + ulp_T(pre)
with hn_c and g_c taken from the oracle's trace of that row (ulp(x): the T
spacing at |x|; ulp_T(pre) at the larger of the two results).
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

import hyper_connection_rank_amd as hc
import oracle
from _util import ulp_dist, ulp_of

NAMES = ("streams", "norm_scale", "down_weight", "up_weight", "inject_weight",
         "prev_block_output", "prev_post_gate")


def args_of(t: Dict[str, torch.Tensor]):
    return tuple(t.get(n) for n in NAMES)


def gpu_run(t: Dict[str, torch.Tensor], attrs: dict, path="auto", want_streams_out=True, device="cuda"):
    g = {k: v.to(device) for k, v in t.items()}
    out = hc.block(*args_of(g), **attrs, want_streams_out=want_streams_out, path=path)
    torch.cuda.synchronize()
    return tuple(None if o is None else o.cpu() for o in out)


class OracleOut(tuple):
    """The oracle's (pre_output, post_gate, streams_out, mag), keeping the
    inputs and attributes so that a judge can trace single rows."""
    inputs: Dict[str, torch.Tensor]
    attrs: dict


def oracle_run(t: Dict[str, torch.Tensor], attrs: dict):
    out = OracleOut(oracle.run(*args_of(t), **attrs, want_mag=True))
    out.inputs, out.attrs = t, attrs
    return out


# Rows beyond this many among the failing elements are not traced (they stay failures).
FLIP_ROWS = 64


def flip_bound(t: Dict[str, torch.Tensor], attrs: dict, flat: torch.Tensor, H: int, pre_g: torch.Tensor,
               pre_o: torch.Tensor) -> Optional[torch.Tensor]:
    """The bound of the last judgement for the pre_output elements at flat
    indices `flat` (into [rows, H]), or None with too many rows to trace."""
    rows = torch.div(flat, H, rounding_mode="floor")
    uniq = torch.unique(rows)
    if uniq.numel() > FLIP_ROWS:
        return None
    dt = pre_o.dtype
    C = int(attrs["num_branches"])
    rs = abs(float(attrs.get("reduction_scale", 1.0)))
    bound = torch.empty(flat.numel(), dtype=torch.float64)
    for r in uniq.tolist():
        one = {k: (v[r:r + 1].contiguous() if k in ("streams", "prev_block_output", "prev_post_gate") else v)
               for k, v in t.items()}
        tr = oracle.trace(*args_of(one), row=0, **attrs)
        hn = tr["hn"].double().view(C, H)
        g = tr["g"].double().view(C, H)
        uh, ug = ulp_of(hn, dt), ulp_of(g, dt)
        step = rs * (uh * g.abs() + hn.abs() * ug + uh * ug).sum(0)
        sel = rows == r
        h = flat[sel] - r * H
        top = torch.maximum(pre_g.view(-1)[flat[sel]].double().abs(), pre_o.view(-1)[flat[sel]].double().abs())
        bound[sel] = step[h] + ulp_of(top, dt)
    return bound


@dataclass
class Judgement:
    name: str
    n: int = 0
    exact: int = 0
    max_ulp: int = 0
    rejudged: int = 0
    bad: int = 0
    worst: str = ""
    extra: dict = field(default_factory=dict)

    def summary(self) -> str:
        frac = self.exact / self.n if self.n else 1.0
        flips = f" (of them by the factor-step bound: {self.extra['flip_judged']})" if "flip_judged" in self.extra else ""
        return (f"{self.name}: n={self.n} exact={frac:.4%} max_ulp={self.max_ulp} "
                f"rejudged={self.rejudged}{flips} bad={self.bad} {self.worst}")


def judge(name: str, gpu: torch.Tensor, ora: torch.Tensor, mag: Optional[torch.Tensor] = None,
          exact: bool = False, last=None) -> Judgement:
    """last(flat indices) -> bounds (or None): the final judgement of elements
    that fail the first two."""
    assert gpu.shape == ora.shape and gpu.dtype == ora.dtype, (gpu.shape, ora.shape, gpu.dtype, ora.dtype)
    j = Judgement(name, n=gpu.numel())
    j.extra["dtype"] = gpu.dtype
    if gpu.numel() == 0:
        return j
    dt = gpu.dtype
    if dt == torch.float32:
        g, o = gpu.double(), ora.double()
        m = o.abs() if mag is None else torch.maximum(o.abs(), mag.double())
        err = (g - o).abs()
        d = ulp_dist(gpu, ora)
        j.exact = int((d == 0).sum())
        j.max_ulp = int(d.max())
        tol = 0.0 if exact else 1e-5
        badmask = err > tol * m
        j.bad = int(badmask.sum())
        if j.bad:
            i = int(torch.argmax((err / torch.clamp(m, min=1e-30)).view(-1)))
            j.worst = f"worst idx {i}: gpu {g.view(-1)[i].item()!r} ora {o.view(-1)[i].item()!r}"
        return j
    d = ulp_dist(gpu, ora)
    j.exact = int((d == 0).sum())
    j.max_ulp = int(d.max())
    if exact:
        j.bad = int((d != 0).sum())
    else:
        fail = d > 2
        if bool(fail.any()):
            m = ora.double().abs() if mag is None else mag.double()
            err = (gpu.double() - ora.double()).abs()
            u = ulp_of(m, dt)
            ok2 = err <= 2 * u
            if last is not None and bool((fail & ~ok2).any()):
                flat = torch.nonzero((fail & ~ok2).view(-1)).view(-1)
                b = last(flat)
                if b is not None:
                    ok3 = err.view(-1)[flat] <= b
                    j.extra["flip_judged"] = int(ok3.sum())
                    ok2 = ok2.clone()
                    ok2.view(-1)[flat[ok3]] = True
            j.rejudged = int((fail & ok2).sum())
            j.bad = int((fail & ~ok2).sum())
            if j.bad:
                # the failing element furthest outside the re-judge bound
                i = int(torch.argmax(torch.where(fail & ~ok2, err / u, torch.zeros_like(err)).view(-1)))
                j.worst = (f"worst idx {i}: gpu {gpu.view(-1)[i].item()!r} ora {ora.view(-1)[i].item()!r} "
                           f"ulp {int(d.view(-1)[i])} err {err.view(-1)[i].item():.3g} = "
                           f"{(err / u).view(-1)[i].item():.2f} ulp of mag {m.view(-1)[i].item():.4g}")
    if j.bad and not j.worst:
        i = int(torch.argmax(d.view(-1)))
        j.worst = (f"worst idx {i}: gpu {gpu.view(-1)[i].item()!r} ora {ora.view(-1)[i].item()!r} "
                   f"ulp {int(d.view(-1)[i])}")
    return j


def judge_block(gpu_out, ora_out, streams_out_expected=True):
    pre_g, post_g, so_g = gpu_out
    pre_o, post_o, so_o, mag = ora_out
    last = None
    if getattr(ora_out, "inputs", None) is not None and pre_o.dim() == 2:
        last = lambda flat: flip_bound(ora_out.inputs, ora_out.attrs, flat, pre_o.shape[1], pre_g, pre_o)  # noqa: E731
    js = [judge("pre_output", pre_g, pre_o, mag=mag, last=last), judge("post_gate", post_g, post_o)]
    if streams_out_expected and so_g is not None:
        js.append(judge("streams_out", so_g, so_o, exact=True))
    return js


# Caps on how far agreement may fall, per workload (name prefix) and else per
# element type: the largest share of pre_output elements that may pass only by
# the cancellation re-judge, and the smallest share that must be bit-exact.
# They sit at about twice the measured shares (decode bf16 1.2 % re-judged and
# 94 % exact; prefill bf16 0.43 % and 96.9 %; wide fp16 2.7 % and 85.8 %; the
# 96-block chain at most 0.7 % and 95.6 %), so a change that moves agreement
# materially fails even when every element still meets the tolerance. They
# apply where pre_output has at least 1000 elements (smaller counts are too
# coarse for a share). post_gate needs no re-judge anywhere.
CAPS = {
    "decode bf16": (0.025, 0.90),
    "decode chain bf16": (0.015, 0.92),
    "prefill bf16": (0.01, 0.94),
    "wide fp16": (0.05, 0.80),
}
DTYPE_CAPS = {torch.bfloat16: (0.025, 0.90), torch.float16: (0.05, 0.80)}


def caps_for(label: str, dtype) -> Optional[tuple]:
    for prefix, cap in CAPS.items():
        if label.startswith(prefix):
            return cap
    return DTYPE_CAPS.get(dtype)


def assert_parity(js, label=""):
    lines = [f"[{label}] " + j.summary() for j in js]
    print("\n".join(lines), flush=True)
    log = os.environ.get("HCLRMIX_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write("\n".join(lines) + "\n")
    assert all(j.bad == 0 for j in js), "\n".join(lines)
    for j in js:
        if j.name == "post_gate":
            assert j.rejudged == 0, "\n".join(lines)
        cap = caps_for(label, j.extra.get("dtype"))
        if j.name == "pre_output" and cap and j.n >= 1000:
            assert j.rejudged <= cap[0] * j.n, f"re-judged share above {cap[0]:.1%}: " + "\n".join(lines)
            assert j.exact >= cap[1] * j.n, f"bit-exact share below {cap[1]:.0%}: " + "\n".join(lines)
