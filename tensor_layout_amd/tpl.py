"""Thin ctypes binding of libtpl.so (argument marshalling only).

The names follow the C ABI in include/tpl.h: ``tpl_permute``,
``tpl_permute_swizzled``, ``tpl_permute_staged``, ``tpl_plan`` (with the
swizzled form behind its keyword arguments), ``tpl_status_string`` and
``tpl_last_error``.  ``PreparedPermute`` marshals one layout once for
repeated calls.  Two conveniences take torch tensors: ``permute`` (flat
storage plus explicit extents and strides; it checks dtypes, extents and
byte ranges) and ``copy_view`` (both layouts read off two views of one
shape); both call ``tpl_permute`` on the tensors' device pointers and
torch's current stream.  Every step of the permutation runs in the
library's HIP kernels; if the library is missing or cannot be loaded every
call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# TPL_LIBRARY names another build of the same library to load instead (the
# tests' host-only sanitizer build uses it).
LIB_PATH = os.environ.get("TPL_LIBRARY") or os.path.join(HERE, "libtpl.so")

TPL_OK = 0
TPL_E_ARG = 1
TPL_E_DTYPE_WIDTH = 2
TPL_E_DTYPE = 3
TPL_E_EXTENT = 4
TPL_E_LAYOUT = 5
TPL_E_NO_K = 6
TPL_E_ALIAS = 7
TPL_E_HIP = 8

TPL_GEOM_GFX950 = 0
TPL_GEOM_PAGES32 = 1
TPL_GEOM_GFX950_HALFWAVE = 2
TPL_GEOM_GFX950_INPLACE = 3

KERNELS = {0: "none", 1: "gather", 2: "quad", 3: "lds", 4: "reg16", 5: "copy", 6: "swap", 7: "rec", 8: "etile"}
MAX_SHARD = 10

EXPORTED = ("tpl_permute", "tpl_plan", "tpl_status_string", "tpl_last_error", "tpl_permute_staged",
            "tpl_permute_swizzled", "tpl_plan_swizzled")


class TplError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class _Swizzle(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("base", ctypes.c_int32), ("shift", ctypes.c_int32)]


def _swz(z):
    """(bits, base, shift) or None -> pointer to a tpl_swizzle (None = plain)."""
    if z is None:
        return None
    return ctypes.byref(_Swizzle(int(z[0]), int(z[1]), int(z[2])))


class _PlanInfo(ctypes.Structure):
    _fields_ = [
        ("status", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("extent", ctypes.c_int64 * MAX_SHARD),
        ("src_str", ctypes.c_int64 * MAX_SHARD),
        ("dst_str", ctypes.c_int64 * MAX_SHARD),
        ("P", ctypes.c_int64),
        ("k", ctypes.c_int32),
        ("shift", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("k_w", ctypes.c_int32),
        ("shift_w", ctypes.c_int32),
        ("mask_w", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("tile", ctypes.c_int32 * 2),
        ("chunks_per_thread", ctypes.c_int32),
        ("lds_pitch", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("block", ctypes.c_int64),
    ]


@dataclass
class PlanInfo:
    status: int
    reason: str
    extent: List[int] = field(default_factory=list)
    src_str: List[int] = field(default_factory=list)
    dst_str: List[int] = field(default_factory=list)
    P: int = 0
    k: int = 0
    shift: int = 0
    mask: int = 0
    k_w: int = 0
    shift_w: int = 0
    mask_w: int = 0
    kernel: str = "none"
    tile: tuple = (0, 0)
    chunks_per_thread: int = 0
    lds_pitch: int = 0
    grid: int = 0
    block: int = 0

    @property
    def ok(self) -> bool:
        return self.status == TPL_OK


_lib = None


def load(path: str = LIB_PATH):
    """Load libtpl.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first (python -c 'import __graft_entry__ as g; g.build()')")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7, and a
    # library loaded before torch would pull in a second copy from /opt/rocm.
    # Loading torch first makes libtpl.so bind to torch's runtime, so device
    # pointers and stream handles from torch are valid in the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.tpl_permute.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                i64p, i64p, i64p, i64p, ctypes.c_int64, ctypes.c_void_p]
    lib.tpl_permute.restype = ctypes.c_int
    zp = ctypes.POINTER(_Swizzle)
    lib.tpl_permute_swizzled.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         i64p, i64p, i64p, i64p, ctypes.c_int64, zp, zp, ctypes.c_void_p]
    lib.tpl_permute_swizzled.restype = ctypes.c_int
    lib.tpl_permute_staged.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       i64p, i64p, i64p, i64p, ctypes.c_int64, zp, zp, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.tpl_permute_staged.restype = ctypes.c_int
    lib.tpl_plan.argtypes = [ctypes.c_int, ctypes.c_int, i64p, i64p, i64p, i64p, ctypes.c_int64,
                             ctypes.c_int, ctypes.POINTER(_PlanInfo)]
    lib.tpl_plan.restype = ctypes.c_int
    lib.tpl_plan_swizzled.argtypes = [ctypes.c_int, ctypes.c_int, i64p, i64p, i64p, i64p, ctypes.c_int64,
                                      zp, zp, ctypes.c_int, ctypes.POINTER(_PlanInfo)]
    lib.tpl_plan_swizzled.restype = ctypes.c_int
    lib.tpl_status_string.argtypes = [ctypes.c_int]
    lib.tpl_status_string.restype = ctypes.c_char_p
    lib.tpl_last_error.argtypes = []
    lib.tpl_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _arr(xs: Sequence[int]):
    return (ctypes.c_int64 * max(1, len(xs)))(*[int(x) for x in xs])


def tpl_status_string(status: int) -> str:
    return load().tpl_status_string(int(status)).decode()


def tpl_last_error() -> str:
    return load().tpl_last_error().decode()


def tpl_permute(src_ptr: int, dst_ptr: int, dtype_bytes: int, extents: Sequence[int],
                src_strides: Sequence[int], dst_strides: Sequence[int],
                elem_offsets: Sequence[int] = (0, 0), batch: int = 1, stream: int = 0) -> int:
    """Call the C entry point on raw device pointers; returns the status code."""
    lib = load()
    return lib.tpl_permute(ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr), int(dtype_bytes),
                           len(extents), _arr(extents), _arr(src_strides), _arr(dst_strides),
                           _arr(elem_offsets), int(batch), ctypes.c_void_p(stream))


def tpl_permute_swizzled(src_ptr: int, dst_ptr: int, dtype_bytes: int, extents: Sequence[int],
                         src_strides: Sequence[int], dst_strides: Sequence[int],
                         elem_offsets: Sequence[int] = (0, 0), batch: int = 1, src_swizzle=None,
                         dst_swizzle=None, stream: int = 0) -> int:
    """tpl_permute with swizzled operands; a swizzle is (bits, base, shift) or None."""
    lib = load()
    return lib.tpl_permute_swizzled(ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr), int(dtype_bytes),
                                    len(extents), _arr(extents), _arr(src_strides), _arr(dst_strides),
                                    _arr(elem_offsets), int(batch), _swz(src_swizzle), _swz(dst_swizzle),
                                    ctypes.c_void_p(stream))


class PreparedPermute:
    """tpl_permute (or tpl_permute_swizzled) with the layout arguments marshalled once.

    Calling the object with (src_ptr, dst_ptr, stream) makes the same C call
    as tpl_permute(src_ptr, dst_ptr, dtype_bytes, extents, ...), without
    rebuilding the ctypes arrays each time; it returns the status code.
    """

    def __init__(self, dtype_bytes: int, extents: Sequence[int], src_strides: Sequence[int],
                 dst_strides: Sequence[int], elem_offsets: Sequence[int] = (0, 0), batch: int = 1,
                 src_swizzle=None, dst_swizzle=None):
        lib = load()
        self._args = (int(dtype_bytes), len(extents), _arr(extents), _arr(src_strides), _arr(dst_strides),
                      _arr(elem_offsets), int(batch))
        if src_swizzle is None and dst_swizzle is None:
            self._fn = lib.tpl_permute
            self._swz = ()
        else:
            self._fn = lib.tpl_permute_swizzled
            self._zs = _Swizzle(*src_swizzle) if src_swizzle is not None else None
            self._zd = _Swizzle(*dst_swizzle) if dst_swizzle is not None else None
            self._swz = (ctypes.byref(self._zs) if self._zs is not None else None,
                         ctypes.byref(self._zd) if self._zd is not None else None)

    def __call__(self, src_ptr: int, dst_ptr: int, stream: int = 0) -> int:
        w, rank, e, s, d, o, b = self._args
        return self._fn(src_ptr, dst_ptr, w, rank, e, s, d, o, b, *self._swz, stream)


def tpl_permute_staged(src_ptr: int, dst_ptr: int, dtype_bytes: int, extents: Sequence[int],
                       src_strides: Sequence[int], dst_strides: Sequence[int],
                       elem_offsets: Sequence[int] = (0, 0), batch: int = 1, xor_k: int = -1,
                       stream: int = 0, src_swizzle=None, dst_swizzle=None) -> int:
    """Call the staged (one batch item per half-wave, through LDS) entry point."""
    lib = load()
    return lib.tpl_permute_staged(ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr), int(dtype_bytes),
                                  len(extents), _arr(extents), _arr(src_strides), _arr(dst_strides),
                                  _arr(elem_offsets), int(batch), _swz(src_swizzle), _swz(dst_swizzle),
                                  int(xor_k), ctypes.c_void_p(stream))


def tpl_plan(dtype_bytes: int, extents: Sequence[int], src_strides: Sequence[int],
             dst_strides: Sequence[int], elem_offsets: Optional[Sequence[int]] = None,
             batch: int = 1, geometry: int = TPL_GEOM_GFX950, src_swizzle=None,
             dst_swizzle=None) -> PlanInfo:
    """Host-only planning (no GPU needed); with swizzles it calls tpl_plan_swizzled."""
    lib = load()
    info = _PlanInfo()
    offs = _arr(elem_offsets) if elem_offsets is not None else None
    if src_swizzle is None and dst_swizzle is None:
        st = lib.tpl_plan(int(dtype_bytes), len(extents), _arr(extents), _arr(src_strides),
                          _arr(dst_strides), offs, int(batch), int(geometry), ctypes.byref(info))
    else:
        st = lib.tpl_plan_swizzled(int(dtype_bytes), len(extents), _arr(extents), _arr(src_strides),
                                   _arr(dst_strides), offs, int(batch), _swz(src_swizzle), _swz(dst_swizzle),
                                   int(geometry), ctypes.byref(info))
    reason = tpl_last_error() if st != TPL_OK else ""
    r = info.rank
    return PlanInfo(st, reason, list(info.extent[:r]), list(info.src_str[:r]), list(info.dst_str[:r]),
                    info.P, info.k, info.shift, info.mask, info.k_w, info.shift_w, info.mask_w,
                    KERNELS.get(info.kernel, "?"), (info.tile[0], info.tile[1]), info.chunks_per_thread,
                    info.lds_pitch,
                    info.grid, info.block)


def _cosize(extents, strides):
    if any(e == 0 for e in extents):
        return 0
    return 1 + sum((e - 1) * s for e, s in zip(extents, strides))


def _swz_reach(n_elems, z):
    """A bound on one past the largest swizzled offset of offsets 0 .. n_elems - 1:
    the swizzle rewrites only bits below base + bits."""
    if z is None or z[0] == 0 or n_elems == 0:
        return n_elems
    return ((n_elems - 1) | ((1 << (z[1] + z[0])) - 1)) + 1


def copy_view(dst, src, stream=None) -> None:
    """Copy the strided tensor view ``src`` into the view ``dst`` (same shape
    and dtype): every element lands where ``dst``'s own strides put it, as
    ``dst[i, j, ...] = src[i, j, ...]``.  The layouts are the views' sizes
    and strides, the bases their data pointers (storage offsets included),
    so transposed, permuted, sliced and broadcast (stride-0) sources and
    transposed or sliced destinations all map onto one tpl_permute call.
    Size-1 dimensions are dropped (they move no address).  A destination
    that overlaps the source is the library's case: a square transpose onto
    itself runs in place, other overlaps raise TplError(TPL_E_ALIAS).
    Raises TplError on any non-OK status."""
    import torch

    if tuple(src.shape) != tuple(dst.shape):
        raise TplError(TPL_E_EXTENT, "extent mismatch")
    if src.dtype != dst.dtype:
        raise TplError(TPL_E_DTYPE, "dtype mismatch")
    if not (src.is_cuda and dst.is_cuda):
        raise TplError(TPL_E_ARG, "tensors must live on the GPU")
    dims = [i for i, e in enumerate(src.shape) if e != 1]
    if src.numel() == 0:
        return
    ext = tuple(int(src.shape[i]) for i in dims) or (1,)
    ss = tuple(int(src.stride(i)) for i in dims) or (1,)
    ds = tuple(int(dst.stride(i)) for i in dims) or (1,)
    if stream is None:
        stream = torch.cuda.current_stream(src.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = tpl_permute(src.data_ptr(), dst.data_ptr(), src.element_size(), ext, ss, ds, (0, 0), 1, sp)
    if st != TPL_OK:
        raise TplError(st, tpl_last_error())


def permute(dst, src, extents: Sequence[int], src_strides: Sequence[int], dst_strides: Sequence[int],
            src_offset: int = 0, dst_offset: int = 0, batch: int = 1, dtype_bytes: Optional[int] = None,
            stream=None, src_swizzle=None, dst_swizzle=None) -> None:
    """Permute ``src`` into ``dst`` (torch tensors on the GPU, used as flat storage).

    Argument order is (dst, src) as in the pages' ``permute_layout(dst, src)``.
    Strides and offsets are in elements of ``dtype_bytes`` bytes (default: the
    tensors' element size).  Raises TplError on any non-OK status.
    """
    import torch

    if src.dtype != dst.dtype and dtype_bytes is None:
        raise TplError(TPL_E_DTYPE, "dtype mismatch")
    w = int(dtype_bytes or src.element_size())
    if not (src.is_cuda and dst.is_cuda):
        raise TplError(TPL_E_ARG, "tensors must live on the GPU")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise TplError(TPL_E_ARG, "tensors must be contiguous storage")
    if not (len(extents) == len(src_strides) == len(dst_strides)):
        raise TplError(TPL_E_EXTENT, "extent mismatch")
    n = batch
    for e in extents:
        n *= e
    if n > 0:
        need_s = (src_offset + _swz_reach(batch * _cosize(extents, src_strides), src_swizzle)) * w
        need_d = (dst_offset + _swz_reach(batch * _cosize(extents, dst_strides), dst_swizzle)) * w
        if need_s > src.numel() * src.element_size() or need_d > dst.numel() * dst.element_size():
            raise TplError(TPL_E_ARG, "layout reaches past the end of a tensor")
    if stream is None:
        stream = torch.cuda.current_stream(src.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if src_swizzle is None and dst_swizzle is None:
        st = tpl_permute(src.data_ptr(), dst.data_ptr(), w, extents, src_strides, dst_strides,
                         (src_offset, dst_offset), batch, sp)
    else:
        st = tpl_permute_swizzled(src.data_ptr(), dst.data_ptr(), w, extents, src_strides, dst_strides,
                                  (src_offset, dst_offset), batch, src_swizzle, dst_swizzle, sp)
    if st != TPL_OK:
        raise TplError(st, tpl_last_error())
