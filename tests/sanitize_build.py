"""Build the library with AddressSanitizer and UndefinedBehaviorSanitizer on
its host code (the planner, the plan cache and the C entry points); the
device code is compiled as usual, without sanitizers.  Used by
test_sanitize_host.py, which loads the result in a child process through
TPL_LIBRARY with the sanitizer runtime preloaded.  Runs on the CPU only."""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

from tensor_layout_amd import build

SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The clang ASan runtime shared object (it carries the UBSan handlers too)."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(build.HIPCC)), "..", "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found")
    return os.path.realpath(hits[-1])


def build_sanitized(outdir: str) -> str:
    # Host code at -O1 with debug info; device code as in the library build
    # (-O3, no debug info), which keeps the build to about 45 s on 8 cores.
    flags = [f for f in build.FLAGS if f != "-shared"] + ["-Xarch_host", "-O1", "-Xarch_host", "-g"] + SAN_FLAGS
    objs = [os.path.join(outdir, s + ".o") for s in build.SOURCES]
    jobs = [[build.HIPCC] + flags + ["-c", os.path.join(build.CSRC, s), "-o", o] for s, o in zip(build.SOURCES, objs)]

    def run(cmd):
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"{' '.join(cmd)}\n{res.stderr[-3000:]}")

    with cf.ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        for f in [ex.submit(run, j) for j in jobs]:
            f.result()
    lib = os.path.join(outdir, "libtpl_san.so")
    run([build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
         "-shared-libsan"] + objs + ["-o", lib])
    return lib
