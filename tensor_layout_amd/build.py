"""Build the HIP library libtpl.so in-tree for gfx950 (hipcc cross-compiles; no GPU needed)."""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtpl.so")
# One translation unit per kernel family, compiled in parallel.
SOURCES = ["planner.cpp", "kernels.hip", "kernels_stream.hip", "kernels_quad.hip", "kernels_lds.hip",
           "kernels_lds_w12.hip", "kernels_lds_w48.hip", "kernels_lds_w16.hip",
           "kernels_swap.hip", "kernels_rec.hip", "kernels_etile.hip", "staged.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wshadow", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


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
    """Build libtpl.so and the C ABI test client (both in-tree).

    Every source is compiled to an object on its own (in parallel), then the
    objects are linked."""
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objdir = tempfile.mkdtemp(prefix="tpl_build_")
    try:
        objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
        jobs = [[HIPCC] + compile_flags + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    if os.path.exists(CLIENT_SRC):
        ctmp = CLIENT + ".tmp"
        _run([HIPCC, "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), CLIENT_SRC,
              "-L", HERE, "-ltpl", "-Wl,-rpath,$ORIGIN/../../tensor_layout_amd", "-o", ctmp], verbose)
        os.replace(ctmp, CLIENT)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
