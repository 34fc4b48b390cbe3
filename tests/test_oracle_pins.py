"""Pins of the data oracle to things other than itself.

Each pin is a function of a permute implementation with the signature of
``oracle.permute_py``.  The C oracle and the pure-Python statement must pass
every pin; each planted mistake (a mutant of the Python statement, defined
below) must fail at least one of them, which shows the pins can see that kind
of mistake.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, workloads
from tests import goldens


# --------------------------------------------------------------------------
# adapters


def c_impl(src: bytes, dst: bytearray, w, extents, ss, ds, offsets=(0, 0), batch=1):
    s = np.frombuffer(bytes(src), dtype=np.uint8).copy()
    d = np.frombuffer(bytes(dst), dtype=np.uint8).copy()
    oracle.permute(s, d, w, extents, ss, ds, offsets, batch)
    dst[:] = d.tobytes()
    return dst


def c_impl_inplace(buf: bytearray, w, extents, ss, ds, offsets=(0, 0), batch=1):
    a = np.frombuffer(bytes(buf), dtype=np.uint8).copy()
    oracle.permute(a, a, w, extents, ss, ds, offsets, batch)
    buf[:] = a.tobytes()
    return buf


def cosize(extents, strides):
    return 1 + sum((e - 1) * s for e, s in zip(extents, strides))


# --------------------------------------------------------------------------
# pins


def pin_sf_generated_ir(impl) -> bool:
    """permute_layout page, generated IR: B[write(s,r,tx)] == A[read(s,r,tx)]."""
    g = goldens.sf_ir()
    wl = workloads.SF_WORKED
    a = synth.random_bytes(wl.seed, 256 * 4)
    out = bytearray(b"\xa5" * (256 * 4))
    impl(a.tobytes(), out, 4, wl.extents, wl.src_strides, wl.dst_strides)
    A = np.frombuffer(a.tobytes(), dtype=np.uint32)
    B = np.frombuffer(bytes(out), dtype=np.uint32)
    written = set()
    R = g["ranges"]
    for s in range(R["s"]):
        for r in range(R["r"]):
            for tx in range(R["tx"]):
                ri = goldens.eval_index(g["read"], s=s, r=r, tx=tx)
                wi = goldens.eval_index(g["write"], s=s, r=r, tx=tx)
                if B[wi] != A[ri]:
                    return False
                written.add(wi)
    return written == set(range(256))


def pin_address_examples(impl) -> bool:
    """Buffers page, 4x8 example: moving a row-major A into B declared four ways."""
    for name, shape, strides, off, expr in goldens.address_examples():
        n_dst = off + cosize(shape, strides)
        a = synth.random_bytes(0xADD0, 32 * 4)
        out = bytearray(b"\x00" * (n_dst * 4))
        impl(a.tobytes(), out, 4, shape, (8, 1), strides, (0, off), 1)
        A = np.frombuffer(a.tobytes(), dtype=np.uint32)
        B = np.frombuffer(bytes(out), dtype=np.uint32)
        for i in range(shape[0]):
            for j in range(shape[1]):
                if B[goldens.eval_index(expr, i=i, j=j)] != A[i * 8 + j]:
                    return False
    return True


def pin_view_permute(impl) -> bool:
    """Buffers page, view/permute: reading A through each view into a dense buffer."""
    for name, idx, strides, expr in goldens.view_permute_examples():
        shape = (64, 4) if name.startswith("view") else (4, 4)
        a = synth.random_bytes(0x71E3, 256 * 4)
        n = shape[0] * shape[1]
        out = bytearray(b"\x00" * (n * 4))
        impl(a.tobytes(), out, 4, shape, strides, (shape[1], 1), (0, 0), 1)
        A = np.frombuffer(a.tobytes(), dtype=np.uint32)
        B = np.frombuffer(bytes(out), dtype=np.uint32)
        for x in range(shape[0]):
            for y in range(shape[1]):
                if B[x * shape[1] + y] != A[goldens.eval_index(expr, **{idx[0]: x, idx[1]: y})]:
                    return False
    return True


def _np_dtype(w):
    return {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[w]


def pin_numpy_transpose(impl) -> bool:
    """The workloads' layouts on small sizes equal numpy's transpose (a library routine)."""
    cases = [
        # (w, extents, src, dst, batch, numpy shape, axes)
        (4, (4, 32), (32, 1), (1, 4), 8, (8, 4, 32), (0, 2, 1)),
        (2, (128, 64), (64, 1), (1, 128), 2, (2, 128, 64), (0, 2, 1)),
        (2, (16, 8), (8, 1), (1, 16), 3, (3, 16, 8), (0, 2, 1)),
    ]
    for w in (1, 2, 4, 8):
        e = (3, 5, 4, 6)
        src = (5 * 4 * 6, 4 * 6, 6, 1)
        # destination: row-major layout of the permuted shape (e0, e2, e3, e1)
        dst = (e[2] * e[3] * e[1], 1, e[3] * e[1], e[1])
        cases.append((w, e, src, dst, 1, e, (0, 2, 3, 1)))
    cases.append((2, (40, 24), (24, 1), (1, 40), 1, (40, 24), (1, 0)))
    for w, ext, ss, ds, batch, shape, axes in cases:
        n = batch * int(np.prod(ext))
        x = synth.random_bytes(0xC0DE + w, n * w).view(_np_dtype(w)).reshape(shape)
        out = bytearray(b"\x00" * (n * w))
        impl(x.tobytes(), out, w, ext, ss, ds, (0, 0), batch)
        if np.frombuffer(bytes(out), dtype=_np_dtype(w)).tobytes() != np.ascontiguousarray(x.transpose(axes)).tobytes():
            return False
    # 16-byte elements: a (n, n, 4) uint32 view transposed on its first two axes.
    nn = 12
    x = synth.random_bytes(0x16B, nn * nn * 16).view(np.uint32).reshape(nn, nn, 4)
    out = bytearray(b"\x00" * (nn * nn * 16))
    impl(x.tobytes(), out, 16, (nn, nn), (nn, 1), (1, nn), (0, 0), 1)
    return bytes(out) == np.ascontiguousarray(x.transpose(1, 0, 2)).tobytes()


def _strided_expected(src_bytes, dst_init, w, ext, ss, ds, offs, batch):
    """numpy strided views: dst_view[...] = src_view (library address arithmetic)."""
    dt = np.dtype(f"V{w}")
    S = np.frombuffer(src_bytes, dtype=dt)
    D = np.frombuffer(dst_init, dtype=dt).copy()
    shape = (batch,) + tuple(ext)
    sv = np.lib.stride_tricks.as_strided(
        S[offs[0]:], shape=shape, strides=tuple(x * w for x in (cosize(ext, ss),) + tuple(ss)))
    dv = np.lib.stride_tricks.as_strided(
        D[offs[1]:], shape=shape, strides=tuple(x * w for x in (cosize(ext, ds),) + tuple(ds)))
    dv[...] = sv
    return D.tobytes()


def _random_layout(rng, rank):
    ext = [int(rng.integers(1, 5)) for _ in range(rank)]
    order = list(rng.permutation(rank))
    # injective destination: dense row-major of a permuted order, maybe padded
    ds = [0] * rank
    acc = 1
    for ax in reversed(order):
        ds[ax] = acc
        acc *= ext[ax] + int(rng.integers(0, 2))
    ss = [int(rng.integers(0, 7)) for _ in range(rank)]
    return ext, ss, ds


def pin_strided_views(impl) -> bool:
    """Random small layouts with offsets, padding, broadcast reads and a batch."""
    rng = np.random.default_rng(1234)
    for t in range(40):
        rank = int(rng.integers(1, 5))
        w = int(rng.choice([1, 2, 4, 8, 16]))
        ext, ss, ds = _random_layout(rng, rank)
        batch = int(rng.integers(1, 4))
        offs = (int(rng.integers(0, 5)), int(rng.integers(0, 5)))
        n_src = offs[0] + batch * cosize(ext, ss)
        n_dst = offs[1] + batch * cosize(ext, ds)
        src = synth.random_bytes(0x5100 + t, n_src * w).tobytes()
        dst0 = synth.random_bytes(0xD500 + t, n_dst * w).tobytes()
        out = bytearray(dst0)
        impl(src, out, w, ext, ss, ds, offs, batch)
        if bytes(out) != _strided_expected(src, dst0, w, ext, ss, ds, offs, batch):
            return False
    return True


def pin_invariants(impl) -> bool:
    """Bijective layouts: multiset preserved, inverse round trip, identity = memcpy."""
    rng = np.random.default_rng(77)
    for t in range(12):
        rank = int(rng.integers(2, 5))
        w = int(rng.choice([1, 2, 4, 8]))
        ext = [int(rng.integers(2, 5)) for _ in range(rank)]
        def dense(order):
            st = [0] * rank
            acc = 1
            for ax in reversed(order):
                st[ax] = acc
                acc *= ext[ax]
            return st
        ss = dense(list(range(rank)))
        ds = dense(list(rng.permutation(rank)))
        n = int(np.prod(ext))
        x = synth.random_bytes(0x1A7 + t, n * w).tobytes()
        y = bytearray(n * w)
        impl(x, y, w, ext, ss, ds)
        words_in = sorted(x[i:i + w] for i in range(0, len(x), w))
        words_out = sorted(bytes(y[i:i + w]) for i in range(0, len(y), w))
        if words_in != words_out:
            return False
        z = bytearray(n * w)
        impl(bytes(y), z, w, ext, ds, ss)
        if bytes(z) != x:
            return False
        ident = bytearray(n * w)
        impl(x, ident, w, ext, ss, ss)
        if bytes(ident) != x:
            return False
    return True


def pin_inplace(impl_inplace, impl) -> bool:
    """In-place equals out-of-place (the two phases read all, then write all)."""
    for wl in (workloads.SF_WORKED, workloads.scaled(workloads.SF_BATCHED, batch=16)):
        n = wl.elements
        x = synth.random_bytes(wl.seed, n * 4).tobytes()
        ref = bytearray(n * 4)
        impl(x, ref, 4, wl.extents, wl.src_strides, wl.dst_strides, (0, 0), wl.batch)
        buf = bytearray(x)
        impl_inplace(buf, 4, wl.extents, wl.src_strides, wl.dst_strides, (0, 0), wl.batch)
        if bytes(buf) != bytes(ref):
            return False
    return True


PINS = [pin_sf_generated_ir, pin_address_examples, pin_view_permute, pin_numpy_transpose,
        pin_strided_views, pin_invariants]


# --------------------------------------------------------------------------
# the oracle passes


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_c_oracle_passes(pin):
    assert pin(c_impl)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_python_statement_passes(pin):
    assert pin(oracle.permute_py)


def test_inplace_c_oracle():
    assert pin_inplace(c_impl_inplace, c_impl)


def test_inplace_python_statement():
    def py_inplace(buf, *a):
        return oracle.permute_py(buf, buf, *a)
    assert pin_inplace(py_inplace, oracle.permute_py)


def test_address_rule_examples():
    """Buffers page address rule: data + elem_offset + layout offset of the coordinate."""
    for name, shape, strides, off, expr in goldens.address_examples():
        for i in range(shape[0]):
            for j in range(shape[1]):
                assert oracle.address((i, j), strides, off) == goldens.eval_index(expr, i=i, j=j), name
    for name, idx, strides, expr in goldens.view_permute_examples():
        for x in range(4):
            for y in range(4):
                assert oracle.address((x, y), strides) == goldens.eval_index(expr, **{idx[0]: x, idx[1]: y})


def test_brute_force_axis_orders():
    """Every axis order of small dense tensors (rank <= 4, extents <= 4) vs numpy."""
    shapes = [(3,), (2, 3), (3, 4), (2, 3, 4), (2, 2, 3, 2), (4, 1, 3, 2)]
    for shape in shapes:
        rank = len(shape)
        x = synth.random_bytes(0xB0 + rank, int(np.prod(shape)) * 2).view(np.uint16).reshape(shape)
        src = [int(np.prod(shape[i + 1:])) for i in range(rank)]
        for axes in itertools.permutations(range(rank)):
            # dst = row-major layout of the permuted shape: stride of source axis axes[k]
            pshape = [shape[a] for a in axes]
            dst = [0] * rank
            for k, a in enumerate(axes):
                dst[a] = int(np.prod(pshape[k + 1:]))
            out = np.zeros(x.size, dtype=np.uint16)
            oracle.permute(x.reshape(-1).view(np.uint8), out.view(np.uint8), 2, shape, src, dst)
            assert out.tobytes() == np.ascontiguousarray(x.transpose(axes)).tobytes(), (shape, axes)


def test_special_encodings_survive():
    """fp32 NaN payloads, sNaN, -0, Inf and denormals come through bit for bit."""
    wl = workloads.scaled(workloads.SF_BATCHED, batch=64)
    x = synth.random_bytes(wl.seed, wl.elements * 4).view(np.uint32).copy()
    synth.inject_f32_specials(x, wl.seed ^ 0x55, rate_log2=2)
    assert np.isin(synth.F32_SPECIALS, x).all()
    out = np.zeros_like(x)
    oracle.permute(x.view(np.uint8), out.view(np.uint8), 4, wl.extents, wl.src_strides,
                   wl.dst_strides, (0, 0), wl.batch)
    assert out.tobytes() == np.ascontiguousarray(x.reshape(64, 4, 32).transpose(0, 2, 1)).tobytes()


def test_empty_and_zero_batch():
    x = np.arange(16, dtype=np.uint8)
    y = np.full(16, 0xA5, dtype=np.uint8)
    oracle.permute(x, y, 1, (0, 4), (4, 1), (1, 4))
    oracle.permute(x, y, 1, (4, 4), (4, 1), (1, 4), batch=0)
    assert (y == 0xA5).all()


def test_out_of_range_is_refused():
    x = np.arange(16, dtype=np.uint8)
    y = np.zeros(15, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.permute(x, y, 1, (4, 4), (4, 1), (1, 4))


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by some pin


def _generic(src, dst, w, extents, ss, ds, offsets=(0, 0), batch=1, *, snapshot=True,
             dense_span=False, nbytes=None, rev_src=False, drop_offsets=False):
    def span(st):
        if dense_span:
            return int(np.prod(extents))
        return cosize(extents, st)
    src = bytes(src) if snapshot else src
    if drop_offsets:
        offsets = (0, 0)
    nb = w if nbytes is None else nbytes
    total = int(np.prod(extents))
    for b in range(batch):
        for n in range(total):
            coord, rem = [], n
            for e in reversed(extents):
                coord.append(rem % e)
                rem //= e
            coord.reverse()
            cs = coord[::-1] if rev_src else coord
            so = offsets[0] + b * span(ss) + sum(c * s for c, s in zip(cs, ss))
            do = offsets[1] + b * span(ds) + sum(c * s for c, s in zip(coord, ds))
            dst[do * w:do * w + nb] = src[so * w:so * w + nb]
    return dst


MUTANTS = {
    "dropped_offset": lambda *a, **k: _generic(*a, drop_offsets=True, **k),
    "swapped_strides": lambda s, d, w, e, ss, ds, *a, **k: _generic(s, d, w, e, ds, ss, *a, **k),
    "dense_batch_span": lambda *a, **k: _generic(*a, dense_span=True, **k),
    "first_byte_only": lambda *a, **k: _generic(*a, nbytes=1, **k),
    "reversed_src_coords": lambda *a, **k: _generic(*a, rev_src=True, **k),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mutant = MUTANTS[name]
    assert not all(pin(mutant) for pin in PINS), name


def test_missing_snapshot_is_caught():
    def inplace_no_snapshot(buf, w, e, ss, ds, offs=(0, 0), batch=1):
        return _generic(buf, buf, w, e, ss, ds, offs, batch, snapshot=False)
    assert not pin_inplace(inplace_no_snapshot, oracle.permute_py)
