"""GPU parity of the standalone inv_rms (FreeToken PR #101, "compute the
hyper-connection pre-norm in one kernel"): hclrmix_inv_rms through the C-ABI
against the CPU oracle (fp64, one rounding to fp32), over shapes, element
types, leading dimensions, magnitudes, the unaligned path and the page's full
size; plus the page's accuracy floor (section "Accuracy") on the GPU result."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import hyper_connection_rank_amd as hc
import oracle

pytestmark = pytest.mark.gpu

T_OF = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _ulps(a, b):
    ia = a.view(torch.int32).to(torch.int64)
    ib = b.view(torch.int32).to(torch.int64)
    ia = torch.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = torch.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return (ia - ib).abs()


def _check(x_cpu, eps, label):
    got = hc.hclrmix_inv_rms(x_cpu.cuda(), eps).cpu()
    ref = oracle.inv_rms(x_cpu.reshape(-1, x_cpu.shape[-1]).contiguous(), eps)
    d = _ulps(got, ref)
    assert d.max().item() <= 1, (label, d.max().item())
    assert (d > 0).float().mean().item() <= 1e-3, label
    return got


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(T_OF[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,dim", [(1, 1), (3, 7), (2, 9), (5, 16384), (33, 2560), (17, 10240), (4, 40000)])
def test_inv_rms_shapes(dtype, rows, dim):
    _check(_rand((rows, dim), dtype, 100 + rows + dim), 1e-6, (dtype, rows, dim))


def test_inv_rms_leading_dims_flatten():
    """x [B, S, hc, D] reduces over hc*D per (b, s), as the page's flatten(2)."""
    x = _rand((2, 3, 4, 256), "bf16", 9)
    got = _check(x.reshape(2, 3, 4 * 256), 1e-6, "leading")
    assert got.shape == (6,)


@pytest.mark.parametrize("dtype,scales", [("bf16", (2.0 ** -60, 2.0 ** -20, 2.0 ** 20, 2.0 ** 60)),
                                          ("f32", (2.0 ** -60, 2.0 ** 60)), ("f16", (2.0 ** -8, 2.0 ** 8))])
def test_inv_rms_magnitude_range(dtype, scales):
    """Squares beyond the fp32 range (or below it) are exact in the fp64 sum."""
    for s in scales:
        _check(_rand((16, 4096), dtype, 21, s), 0.0, (dtype, s))


def test_inv_rms_unaligned_start():
    """A row start that is not 16-byte aligned takes the element-wise path."""
    x = _rand((9, 1025), "bf16", 5)
    got = hc.hclrmix_inv_rms(x.cuda().reshape(-1)[1:].reshape(8, 1153)[:, :].contiguous(), 1e-6).cpu()
    ref = oracle.inv_rms(x.reshape(-1)[1:].reshape(8, 1153).contiguous(), 1e-6)
    assert _ulps(got, ref).max().item() <= 1
    buf = x.cuda().reshape(-1)
    sub = buf[1:1 + 8 * 1024].view(8, 1024)  # data_ptr 2 bytes past a 16-byte boundary
    got = hc.hclrmix_inv_rms(sub, 1e-6).cpu()
    ref = oracle.inv_rms(x.reshape(-1)[1:1 + 8 * 1024].reshape(8, 1024).contiguous(), 1e-6)
    assert _ulps(got, ref).max().item() <= 1


def test_inv_rms_full_size_and_accuracy_floor():
    """The page's full size (8192 rows, hc_dim 16384, bf16) against the oracle,
    and the GPU result's mean relative error against fp64 at or below the
    page's 3.65e-8 (section "Accuracy")."""
    x = _rand((8192, 16384), "bf16", 1234)
    got = _check(x, 1e-6, "full")
    ref64 = oracle.inv_rms(x, 1e-6, fp64=True)
    rel = ((got.double() - ref64).abs() / ref64).mean().item()
    assert rel <= 3.65e-8, rel


def test_inv_rms_zero_rows_and_row_of_zeros():
    x = torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda")
    assert hc.hclrmix_inv_rms(x, 1e-6).numel() == 0
    z = torch.zeros(3, 64, dtype=torch.bfloat16)
    got = hc.hclrmix_inv_rms(z.cuda(), 0.25).cpu()
    assert torch.equal(got, torch.full((3,), 2.0))
