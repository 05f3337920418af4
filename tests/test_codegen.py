"""Checks on the device code the compiler writes for gfx950 (CPU only: the
sources are compiled to assembly here, nothing runs on a GPU).

The forward kernels issue their direct-to-LDS loads from inline assembly.  On
this architecture a memory instruction may read a scalar register written by
a vector instruction (v_readlane, v_readfirstlane, ...) only five wait states
later, and the compiler inserts no wait before an instruction it cannot see
inside an asm block; a descriptor reloaded just before such a load would be
read stale.  The test compiles the sources that issue them and checks every
such load.
"""
import os
import re
import subprocess
import tempfile

import pytest

from scaled_dot_product_attn_amd import _build

VMEM_SGPR_WAIT_STATES = 5


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _hazards(asm_lines):
    """(kernel, load, writer, wait states) for each direct-to-LDS buffer load
    that reads a scalar register a vector instruction wrote too recently."""
    out, kern = [], None
    for n, line in enumerate(asm_lines):
        if re.match(r"^_Z\w+:", line):
            kern = line.split(":")[0]
        t = line.strip()
        if not (t.startswith("buffer_load") and t.endswith(" lds")):
            continue
        regs = _sgprs(t.split(None, 1)[1].split(",")[1].strip())
        ws, k = 0, n - 1
        while k >= 0 and ws < VMEM_SGPR_WAIT_STATES:
            p = asm_lines[k].strip()
            k -= 1
            if not p or p.startswith((";", ".")) or p.endswith(":"):
                continue
            if p.startswith("s_nop"):
                ws += int(p.split()[1], 0) + 1
                continue
            if p.startswith("v_") and _sgprs(p.split(None, 1)[1].split(",")[0].strip()) & regs:
                out.append((kern, t, p, ws))
            ws += 1
    return out


def test_hazard_scan_finds_a_planted_case():
    asm = ["_Zk:", "  v_readlane_b32 s7, v3, 1", "  s_nop 0",
           "  buffer_load_dwordx4 v1, s[4:7], 0 offen lds"]
    assert len(_hazards(asm)) == 1
    asm[2] = "  s_nop 4"
    assert _hazards(asm) == []


@pytest.mark.timeout(600)
@pytest.mark.parametrize("source", ["attn_fwd_bf16.hip", "attn_bwd.hip"])
def test_direct_to_lds_loads_wait_for_scalar_operands(source):
    src = os.path.join(_build.CSRC, source)
    flags = [f for f in _build.CFLAGS if f != "-fPIC"]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        subprocess.run([_build.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out],
                       check=True, capture_output=True)
        lines = open(out).read().split("\n")
    assert sum(1 for x in lines if x.strip().endswith(" lds")) > 0
    bad = _hazards(lines)
    assert not bad, f"{len(bad)} loads read a scalar register too soon, e.g. {bad[0]}"
