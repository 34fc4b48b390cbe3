"""Build the HIP library libtpl.so in-tree for gfx950 (hipcc cross-compiles; no GPU needed)."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtpl.so")
SOURCES = ["planner.cpp", "kernels.hip", "staged.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wshadow", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


PROBE = os.path.join(HERE, "lds_probe")
PROBE_FLAGS = [f for f in FLAGS if f not in ("-fPIC", "-shared")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    if verbose and msgs:
        print("\n".join(msgs))


# A plain C++ client of the C ABI used by the tests (host code only, links the library).
CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_client.cpp")
CLIENT = os.path.join(ROOT, "tests", "c_abi", "abi_client")


def build(verbose: bool = False) -> str:
    """Build libtpl.so, the LDS bank-geometry probe and the C ABI test client (all in-tree)."""
    tmp = LIB + ".tmp"
    _run([HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    ptmp = PROBE + ".tmp"
    _run([HIPCC] + PROBE_FLAGS + [os.path.join(CSRC, "lds_probe.hip"), "-o", ptmp], verbose)
    os.replace(ptmp, PROBE)
    if os.path.exists(CLIENT_SRC):
        ctmp = CLIENT + ".tmp"
        _run([HIPCC, "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), CLIENT_SRC,
              "-L", HERE, "-ltpl", "-Wl,-rpath,$ORIGIN/../../tensor_layout_amd", "-o", ctmp], verbose)
        os.replace(ctmp, CLIENT)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
