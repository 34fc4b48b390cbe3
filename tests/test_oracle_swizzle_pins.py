"""Pins of the oracle's swizzled operands to things other than itself.

A swizzle (bits, base, shift) XORs the bits-wide field of a layout offset
that starts at bit base + shift into the field that starts at bit base; it
acts on the side's layout offset (batch as the outermost mode) before the
element offset is added.  The pins restate it with integer division instead
of shifts and masks, check it against the chunk-XOR-row pattern of
MMA-swizzled fp16 tiles, and check whole permutes against numpy scatters and
gathers.  The C oracle and a Python statement must pass every pin; each
planted mistake must fail at least one.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth


def swz_divmod(bits, base, shift, m):
    """The swizzle restated with division: m = hi | y | mid | z | lo fields."""
    if bits == 0:
        return m
    lo = m % 2 ** base
    z = (m // 2 ** base) % 2 ** bits
    mid = (m // 2 ** (base + bits)) % 2 ** (shift - bits)
    y = (m // 2 ** (base + shift)) % 2 ** bits
    hi = m // 2 ** (base + shift + bits)
    return (((hi * 2 ** bits + y) * 2 ** (shift - bits) + mid) * 2 ** bits + (z ^ y)) * 2 ** base + lo


def cosize(ext, st):
    if any(e == 0 for e in ext):
        return 0
    return 1 + sum((e - 1) * s for e, s in zip(ext, st))


# --------------------------------------------------------------------------
# implementations under test: (src, dst, w, ext, ss, ds, offs, batch, zs, zd) -> dst


def c_impl(src, dst, w, ext, ss, ds, offs, batch, zs, zd):
    s = np.frombuffer(bytes(src), dtype=np.uint8).copy()
    d = np.frombuffer(bytes(dst), dtype=np.uint8).copy()
    oracle.permute(s, d, w, ext, ss, ds, offs, batch, zs, zd)
    dst[:] = d.tobytes()
    return dst


def _py(src, dst, w, ext, ss, ds, offs, batch, zs, zd, *, after_offset=False, per_item=False,
        fields_swapped=False, base_off_by_one=False, src_side_dropped=False):
    def f(z, m):
        if z is None or z[0] == 0:
            return m
        bits, base, shift = z
        if base_off_by_one:
            base += 1
        if fields_swapped:   # the low field XORed into the high one
            return m ^ (((m >> base) & ((1 << bits) - 1)) << (base + shift))
        return m ^ (((m >> (base + shift)) & ((1 << bits) - 1)) << base)

    src = bytes(src)
    span_s, span_d = cosize(ext, ss), cosize(ext, ds)
    if src_side_dropped:
        zs = None
    total = int(np.prod(ext))
    for b in range(batch):
        for n in range(total):
            coord, rem = [], n
            for e in reversed(ext):
                coord.append(rem % e)
                rem //= e
            coord.reverse()
            ls = sum(c * s for c, s in zip(coord, ss))
            ld = sum(c * s for c, s in zip(coord, ds))
            if after_offset:
                so = f(zs, offs[0] + b * span_s + ls)
                do = f(zd, offs[1] + b * span_d + ld)
            elif per_item:
                so = offs[0] + b * span_s + f(zs, ls)
                do = offs[1] + b * span_d + f(zd, ld)
            else:
                so = offs[0] + f(zs, b * span_s + ls)
                do = offs[1] + f(zd, b * span_d + ld)
            dst[do * w:(do + 1) * w] = src[so * w:(so + 1) * w]
    return dst


def py_impl(*a):
    return _py(*a)


# --------------------------------------------------------------------------
# pins


def pin_function_closed_form(impl) -> bool:
    """The swizzle of single offsets (run through a 1-element scatter per offset
    would be slow; the permute of an identity layout covers every offset)."""
    rng = np.random.default_rng(5)
    for bits, base, shift in [(1, 0, 1), (2, 1, 3), (3, 3, 3), (3, 3, 4), (2, 0, 5), (4, 2, 4)]:
        n = 2 ** (base + shift + bits) * 2 + int(rng.integers(0, 7))
        x = np.arange(n, dtype=np.uint32)
        top = max(swz_divmod(bits, base, shift, m) for m in range(n)) + 1
        out = bytearray(b"\xff" * (4 * top))
        impl(x.tobytes(), out, 4, (n,), (1,), (1,), (0, 0), 1, None, (bits, base, shift))
        got = np.frombuffer(bytes(out), dtype=np.uint32)
        for m in range(n):
            if got[swz_divmod(bits, base, shift, m)] != m:
                return False
    return True


def pin_mma_chunk_pattern(impl) -> bool:
    """A 64 x 64 fp16 tile with 128-byte rows under (3, 3, 3): the 16-byte
    chunk c of row r lands at chunk c XOR (r mod 8) of the same row."""
    r_, c_ = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    x = (r_ * 64 + c_).astype(np.uint16)
    out = bytearray(64 * 64 * 2)
    impl(x.tobytes(), out, 2, (64, 64), (64, 1), (64, 1), (0, 0), 1, None, (3, 3, 3))
    got = np.frombuffer(bytes(out), dtype=np.uint16).reshape(64, 64)
    want = np.empty_like(x)
    for r in range(64):
        for c in range(64):
            want[r, ((c // 8) ^ (r % 8)) * 8 + c % 8] = x[r, c]
    return bool(np.array_equal(got, want))


def pin_involution(impl) -> bool:
    """Scatter through a swizzle, then gather through the same swizzle: back to start."""
    n = 4096
    x = synth.random_bytes(0x51, n * 2).copy()
    mid = bytearray(n * 2)
    impl(x.tobytes(), mid, 2, (n,), (1,), (1,), (0, 0), 1, None, (3, 4, 5))
    back = bytearray(n * 2)
    impl(bytes(mid), back, 2, (n,), (1,), (1,), (0, 0), 1, (3, 4, 5), None)
    return bytes(back) == x.tobytes() and bytes(mid) != x.tobytes()


def pin_offsets_and_batch(impl) -> bool:
    """numpy scatter/gather: element offsets are added after the swizzle, and
    the swizzle sees the batch term (item span 100 is not a multiple of the
    swizzle period, so this separates it from swizzling each item alone)."""
    w, n, batch, o_s, o_d = 4, 100, 3, 5, 9
    z = (2, 1, 3)
    x = synth.random_bytes(0x52, (o_s + n * batch) * w).view(np.uint32).copy()
    top = o_d + max(swz_divmod(*z, m) for m in range(n * batch)) + 1
    out = bytearray(b"\x00" * (top * w))
    impl(x.tobytes(), out, w, (n,), (1,), (1,), (o_s, o_d), batch, None, z)
    want = np.zeros(top, dtype=np.uint32)
    for m in range(n * batch):
        want[o_d + swz_divmod(*z, m)] = x[o_s + m]
    if bytes(out) != want.tobytes():
        return False
    # gather side, same numbers
    srcn = o_s + max(swz_divmod(*z, m) for m in range(n * batch)) + 1
    x2 = synth.random_bytes(0x53, srcn * w).view(np.uint32).copy()
    out2 = bytearray(b"\x00" * ((o_d + n * batch) * w))
    impl(x2.tobytes(), out2, w, (n,), (1,), (1,), (o_s, o_d), batch, z, None)
    want2 = np.zeros(o_d + n * batch, dtype=np.uint32)
    for m in range(n * batch):
        want2[o_d + m] = x2[o_s + swz_divmod(*z, m)]
    return bytes(out2) == want2.tobytes()


def pin_transpose_into_swizzled(impl) -> bool:
    """A 32 x 48 u16 transpose into a swizzled column-major tile equals numpy's
    transpose followed by the restated scatter; bits = 0 equals the plain transpose."""
    a, b = 32, 48
    x = synth.random_bytes(0x54, a * b * 2).view(np.uint16).reshape(a, b).copy()
    t = np.ascontiguousarray(x.T).reshape(-1)
    plain = bytearray(a * b * 2)
    impl(x.tobytes(), plain, 2, (a, b), (b, 1), (1, a), (0, 0), 1, None, (0, 0, 0))
    if bytes(plain) != t.tobytes():
        return False
    z = (2, 3, 2)
    out = bytearray(a * b * 2)
    impl(x.tobytes(), out, 2, (a, b), (b, 1), (1, a), (0, 0), 1, None, z)
    want = np.empty_like(t)
    for m in range(a * b):
        want[swz_divmod(*z, m)] = t[m]
    return bytes(out) == want.tobytes()


PINS = [pin_function_closed_form, pin_mma_chunk_pattern, pin_involution, pin_offsets_and_batch,
        pin_transpose_into_swizzled]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_c_oracle_passes(pin):
    assert pin(c_impl)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_python_statement_passes(pin):
    assert pin(py_impl)


def test_swizzle_function_matches_division_form():
    rng = np.random.default_rng(9)
    for _ in range(2000):
        bits = int(rng.integers(1, 5))
        base = int(rng.integers(0, 6))
        shift = int(rng.integers(bits, 8))
        m = int(rng.integers(0, 1 << 40))
        assert oracle.swizzle(bits, base, shift, m) == swz_divmod(bits, base, shift, m)
    assert oracle.swizzle(0, 3, 3, 12345) == 12345


def test_invalid_swizzles_are_refused():
    x = np.zeros(64, dtype=np.uint8)
    y = np.zeros(64, dtype=np.uint8)
    for z in [(2, 0, 1), (-1, 0, 0), (1, -1, 1), (17, 0, 17)]:
        with pytest.raises(ValueError):
            oracle.permute(x, y, 1, (64,), (1,), (1,), (0, 0), 1, None, z)


MUTANTS = {
    "swizzle_after_offset": lambda *a: _py(*a, after_offset=True),
    "swizzle_per_item": lambda *a: _py(*a, per_item=True),
    "fields_swapped": lambda *a: _py(*a, fields_swapped=True),
    "base_off_by_one": lambda *a: _py(*a, base_off_by_one=True),
    "src_swizzle_dropped": lambda *a: _py(*a, src_side_dropped=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    assert not all(pin(MUTANTS[name]) for pin in PINS), name
