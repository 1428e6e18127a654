"""What the decode handoff assumes of the generated gfx950 code, checked on
the CPU (hipcc compiles hc_decode.hip to device assembly; nothing runs).

Workgroups of k_hc_down publish their slice partials with relaxed agent-scope
stores, count themselves on an arrival counter, and the last one reads the
partials back, with relaxed agent-scope loads into registers or direct
global->LDS loads given the same cache-policy bit. Without a release/acquire
pair this is correct only while those accesses carry sc1: stores then write
through the XCD's L2 to the memory side that every XCD sees, and loads miss
the L2 instead of returning a line cached there by an earlier call."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from hyper_connection_rank_amd import build


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    hipcc = build._hipcc()
    if not os.path.exists(hipcc) and shutil.which(hipcc) is None:
        pytest.skip("hipcc is not installed")
    out = tmp_path_factory.mktemp("asm") / "hc_decode.s"
    cmd = [hipcc] + build.FLAGS + ["-x", "hip", "--cuda-device-only", "-S",
                                   os.path.join(build.CSRC, "hc_decode.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm: str, prefix: str):
    found = []
    for m in re.finditer(r"^(%s\S*):" % re.escape(prefix), asm, re.M):
        found.append((m.group(1), asm[m.end():asm.index(".Lfunc_end", m.end())]))
    return found


def _ops(body: str, op: str):
    """Operand/modifier text of every `op` instruction (exact mnemonic)."""
    return re.findall(r"^\s*%s\s([^\n]*)" % re.escape(op), body, re.M)


def test_decode_handoff_accesses_carry_sc1(decode_asm):
    kernels = _kernels(decode_asm, "_ZN2hc9k_hc_down")
    assert len(kernels) >= 2, "no k_hc_down instances in the assembly"
    for name, body in kernels:
        # 32-bit stores in this kernel are the fp32 slice partials and the
        # counter's reset, all agent-scope.
        stores = _ops(body, "global_store_dword")
        assert stores, name
        assert all(re.search(r"\bsc1\b", s) for s in stores), (name, stores)
        # The register path's agent-scope loads of the partials.
        assert any(re.search(r"\bsc1\b", s) for s in _ops(body, "global_load_dword")), name
        # The LDS-staged path: its direct loads carry sc1 (the weight
        # prefetches into LDS do not need it and do not have it).
        assert any(re.search(r"\bsc1\b", s) for s in _ops(body, "global_load_lds_dwordx4")), name
        # One arrival counter update per workgroup, returning the old count.
        adds = _ops(body, "global_atomic_add")
        assert len(adds) == 1 and re.search(r"\bsc0\b", adds[0]), (name, adds)
