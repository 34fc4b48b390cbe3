"""The device-scope 16-byte store (st16_dev) is an asm statement, so the
compiler's hazard recognizer cannot see it.  On gfx950 a store of more than
8 bytes reads its data registers after issue, so a VALU instruction that
writes one of those registers must come at least 2 wait states after the
store (the compiler keeps that distance for its own stores; the asm carries
it as s_nop 1).  Without that wait the swizzled tile path stored wrong bytes
on MI355X.

This compiles the kernels that use it to gfx950 assembly (host only, no GPU)
and checks every such store: the s_nop that follows has an immediate of at
least 1, and walking forward from the store no VALU instruction writes one of
its data registers before 2 wait states have passed (s_nop N counts N + 1,
any other instruction 1; a branch inside the window fails the check, since
its target is not followed)."""

from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from tensor_layout_amd import build

SOURCES = ["kernels_quad.hip", "kernels_stream.hip", "kernels_lds_w48.hip", "kernels_lds_w16.hip"]
WAIT_STATES = 2

_REG_RANGE = re.compile(r"^v\[(\d+):(\d+)\]$")
_REG_ONE = re.compile(r"^v(\d+)$")


def _vregs(op: str):
    """VGPR numbers named by one operand ("v7", "v[4:7]"), else an empty set."""
    op = op.strip()
    m = _REG_RANGE.match(op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _REG_ONE.match(op)
    return {int(m.group(1))} if m else set()


def _operands(line: str):
    parts = line.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def check_scoped_stores(lines):
    """Returns (stores checked, list of violations) for the assembly lines."""
    insts = [l for l in (x.strip() for x in lines) if l and not l.startswith((";", ".")) and not l.endswith(":")]
    violations, checked = [], 0
    for i, line in enumerate(insts):
        if not (line.startswith("global_store_dwordx4") and " sc1" in line):
            continue
        checked += 1
        data = _vregs(_operands(line)[1])
        if len(data) != 4:
            violations.append(("unparsed data registers", line))
            continue
        nxt = insts[i + 1] if i + 1 < len(insts) else ""
        m = re.match(r"s_nop\s+(\d+)", nxt)
        if not m or int(m.group(1)) < WAIT_STATES - 1:
            violations.append(("store not followed by s_nop >= 1", line, nxt))
        waited = 0
        for later in insts[i + 1:]:
            if waited >= WAIT_STATES:
                break
            m = re.match(r"s_nop\s+(\d+)", later)
            if m:
                waited += int(m.group(1)) + 1
                continue
            if later.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
                violations.append(("branch inside the wait window", line, later))
                break
            if later.startswith("v_"):
                ops = _operands(later)
                if ops and _vregs(ops[0]) & data:
                    violations.append(("VALU writes store data within the wait window", line, later))
                    break
            waited += 1
    return checked, violations


def test_checker_catches_missing_wait():
    """The checker itself, on hand-written assembly: a VALU write right after
    the store, or after only s_nop 0, is flagged; after s_nop 1 it is not."""
    store = "global_store_dwordx4 v[2:3], v[4:7], off sc1 nt"
    assert check_scoped_stores([store, "s_nop 1", "v_mov_b32_e32 v5, 0"]) == (1, [])
    assert check_scoped_stores([store, "s_nop 1", "v_mov_b32_e32 v9, 0", "v_mov_b32_e32 v5, 0"]) == (1, [])
    n, bad = check_scoped_stores([store, "s_nop 0", "v_mov_b32_e32 v6, 0"])
    assert n == 1 and any("VALU writes" in v[0] for v in bad) and any("s_nop >= 1" in v[0] for v in bad)
    n, bad = check_scoped_stores([store, "v_lshl_add_u64 v[6:7], v[0:1], 0, v[2:3]"])
    assert n == 1 and any("VALU writes" in v[0] for v in bad)
    n, bad = check_scoped_stores([store, "s_cbranch_scc0 .LBB0_1", "s_nop 1"])
    assert any("branch" in v[0] for v in bad)
    # a VALU write to other registers inside the window is fine
    assert check_scoped_stores([store, "s_nop 1", "v_add_u32_e32 v8, v1, v2"]) == (1, [])


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
@pytest.mark.parametrize("src", SOURCES)
def test_scoped_stores_carry_their_wait(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    res = subprocess.run([build.HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(build.CSRC, src),
                                                  "-o", str(out)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    checked, violations = check_scoped_stores(out.read_text().splitlines())
    assert checked, "no device-scope 16-byte store found"
    assert not violations, violations[:5]
