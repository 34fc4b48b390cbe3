"""ctypes front end of the C oracle, plus a pure-Python statement of it.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_permute.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the C oracle with the host compiler (plain -O2, one thread)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_permute.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, i64p, i64p, i64p, i64p, ctypes.c_int64,
        ]
        lib.oracle_permute.restype = ctypes.c_int
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_permute_swizzled.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, i64p, i64p, i64p, i64p, ctypes.c_int64, i32p, i32p,
        ]
        lib.oracle_permute_swizzled.restype = ctypes.c_int
        lib.oracle_swizzle.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
        lib.oracle_swizzle.restype = ctypes.c_int64
        lib.oracle_address.argtypes = [ctypes.c_int, i64p, i64p, ctypes.c_int64]
        lib.oracle_address.restype = ctypes.c_int64
        _lib = lib
    return _lib


def _i64(xs: Sequence[int]):
    arr = (ctypes.c_int64 * max(1, len(xs)))(*[int(x) for x in xs])
    return arr


def _swz(z):
    if z is None:
        return None
    return (ctypes.c_int32 * 3)(*[int(v) for v in z])


def permute(src: np.ndarray, dst: np.ndarray, w: int, extents, src_strides, dst_strides,
            offsets=(0, 0), batch: int = 1, src_swizzle=None, dst_swizzle=None) -> None:
    """Run the C oracle on two contiguous byte buffers (``dst`` is written in place).

    ``src`` and ``dst`` may be the same array (the oracle snapshots the source).
    A swizzle is (bits, base, shift) or None.
    """
    lib = _load()
    assert src.flags["C_CONTIGUOUS"] and dst.flags["C_CONTIGUOUS"]
    rank = len(extents)
    if src_swizzle is None and dst_swizzle is None:
        rc = lib.oracle_permute(
            src.ctypes.data, src.nbytes, dst.ctypes.data, dst.nbytes, int(w), rank,
            _i64(extents), _i64(src_strides), _i64(dst_strides), _i64(offsets), int(batch),
        )
    else:
        rc = lib.oracle_permute_swizzled(
            src.ctypes.data, src.nbytes, dst.ctypes.data, dst.nbytes, int(w), rank,
            _i64(extents), _i64(src_strides), _i64(dst_strides), _i64(offsets), int(batch),
            _swz(src_swizzle), _swz(dst_swizzle),
        )
    if rc != 0:
        raise ValueError(f"oracle_permute returned {rc}")


def swizzle(bits: int, base: int, shift: int, m: int) -> int:
    """The oracle's swizzle of one layout offset."""
    return int(_load().oracle_swizzle(int(bits), int(base), int(shift), int(m)))


def address(coord, strides, elem_offset: int = 0) -> int:
    """Element offset of ``coord`` under ``strides`` plus ``elem_offset`` (C oracle)."""
    lib = _load()
    return int(lib.oracle_address(len(coord), _i64(coord), _i64(strides), int(elem_offset)))


def permute_py(src: bytes, dst: bytearray, w: int, extents, src_strides, dst_strides,
               offsets=(0, 0), batch: int = 1) -> bytearray:
    """Pure-Python statement of the same definition (small inputs only)."""
    def cosize(strides):
        if any(e == 0 for e in extents):
            return 0
        return 1 + sum((e - 1) * s for e, s in zip(extents, strides))

    src = bytes(src)  # snapshot: read everything before writing anything
    span_s, span_d = cosize(src_strides), cosize(dst_strides)
    total = 1
    for e in extents:
        total *= e
    for b in range(batch):
        for n in range(total):
            coord, rem = [], n
            for e in reversed(extents):
                coord.append(rem % e)
                rem //= e
            coord.reverse()
            so = offsets[0] + b * span_s + sum(c * s for c, s in zip(coord, src_strides))
            do = offsets[1] + b * span_d + sum(c * s for c, s in zip(coord, dst_strides))
            dst[do * w:(do + 1) * w] = src[so * w:(so + 1) * w]
    return dst
