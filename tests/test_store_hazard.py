"""The device-scope 16-byte store (st16_dev) is an asm statement, so the
compiler's hazard recognizer cannot see it: a VALU write to the store's data
registers must stay 2 wait states behind it, which the asm provides itself
with s_nop 1.  Without that wait the swizzled tile path stored wrong bytes on
MI355X.  This compiles the kernels that use it to gfx950 assembly (host only,
no GPU) and checks that every such store is followed by the wait."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from tensor_layout_amd import build

SOURCES = ["kernels_quad.hip", "kernels_stream.hip"]


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
@pytest.mark.parametrize("src", SOURCES)
def test_scoped_stores_carry_their_wait(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    res = subprocess.run([build.HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(build.CSRC, src),
                                                  "-o", str(out)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l.strip() for l in out.read_text().splitlines()]
    scoped = [i for i, l in enumerate(lines) if l.startswith("global_store_dwordx4") and " sc1" in l]
    assert scoped, "no device-scope 16-byte store found"
    for i in scoped:
        assert lines[i + 1].startswith("s_nop"), (src, lines[i], lines[i + 1])
