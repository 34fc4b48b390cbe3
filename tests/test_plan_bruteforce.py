"""Brute-force cross-check of the plan oracle in the pages' geometry.

A second simulator, written apart from oracle/plan_oracle.py, executes the
pages' per-lane program ([permute] "Algorithm" steps 2-3) directly on the
original layout -- no canonicalisation, no regrouping: at unrolled step r
lane l visits iteration n = l + 32 * (r ^ ((l >> shift) & mask)), whose
coordinate is numpy's row-major unravelling of n over the given extents.  It
marks, per pass of lanes, which of the 32 four-byte banks each lane touches
(a w-byte element covers max(1, w/4) consecutive banks; passes are 32, 16
and 8 lanes for elements of at most 4, 8 and 16 bytes: reading A8) and
accepts a step when no bank column holds two lanes.  It tries every k with
2^k dividing P (shift = 5 - k, mask = 2^k - 1) and keeps the smallest that
clears both phases.

Over a family of tiny tiles (every tile shape of 32 P elements for P up to
8, every source and destination axis order, padded and unpadded rows, all
widths) it
must agree with the plan oracle's P, k, shift and mask, and decline exactly
where the oracle does.  Canonicalisation, regrouping and the lane offsets of
the oracle are thus checked against a simulator that never forms a shard.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

from oracle import plan_oracle as po

LANES = 32
BANKS = 32


def offsets(ext, strides, n):
    coords = np.stack(np.unravel_index(n, ext), axis=-1)      # row-major, last axis fastest
    return coords @ np.asarray(strides, dtype=np.int64)


def step_ok(elem_offsets, w):
    per_lane = max(1, w // 4)
    pass_lanes = LANES if w <= 4 else 128 // w
    first_bank = (elem_offsets * w) // 4
    touched = np.zeros((LANES, BANKS), dtype=np.int64)
    for t in range(per_lane):
        touched[np.arange(LANES), (first_bank + t) % BANKS] += 1
    for p0 in range(0, LANES, pass_lanes):
        if (touched[p0:p0 + pass_lanes].sum(axis=0) > 1).any():
            return False
    return True


def brute_plan(w, ext, ss, ds):
    """(P, k, shift, mask), or None when no k clears both phases."""
    total = int(np.prod(ext))
    P = total // LANES
    lane = np.arange(LANES)
    for k in range(6):
        if (1 << k) > P or P % (1 << k):
            continue
        shift, mask = 5 - k, (1 << k) - 1
        ok = True
        for r in range(P):
            n = lane + LANES * (r ^ ((lane >> shift) & mask))
            if not (step_ok(offsets(ext, ss, n), w) and step_ok(offsets(ext, ds, n), w)):
                ok = False
                break
        if ok:
            return P, k, shift, mask
    return None


def row_major(ext, order, pad):
    """Strides of the row-major layout of the axes in `order`, the innermost
    row padded by `pad` elements."""
    st = [0] * len(ext)
    acc = 1
    for i, ax in enumerate(reversed(order)):
        st[ax] = acc
        acc *= ext[ax] + (pad if i == 0 else 0)
    return st


def family():
    shapes = []
    for P in (1, 2, 4, 8):
        n = 32 * P
        for a in (2, 4, 8, 16, 32):
            if n % a == 0 and n // a > 1:
                shapes.append((a, n // a))
        for a, b in ((2, 4), (4, 2), (2, 8), (4, 4)):
            if n % (a * b) == 0 and n // (a * b) > 1:
                shapes.append((a, b, n // (a * b)))
    for ext in shapes:
        for so in itertools.permutations(range(len(ext))):
            for do in itertools.permutations(range(len(ext))):
                for pad_s, pad_d in ((0, 0), (0, 1), (4, 0), (1, 4)):
                    yield ext, row_major(ext, list(so), pad_s), row_major(ext, list(do), pad_d)


CASES = list(family())


def test_family_is_broad():
    assert len(CASES) > 200
    widths_k = set()
    for ext, ss, ds in CASES[::7]:
        for w in (1, 4, 16):
            got = brute_plan(w, ext, ss, ds)
            widths_k.add(None if got is None else got[1])
    # the family reaches declines and several k
    assert None in widths_k and len(widths_k - {None}) >= 3


@pytest.mark.parametrize("w", [1, 2, 4, 8, 16])
def test_bruteforce_agrees_with_plan_oracle(w):
    for ext, ss, ds in CASES:
        want = brute_plan(w, ext, ss, ds)
        p = po.plan(w, ext, ss, ds)
        if want is None:
            assert not p.ok and p.reason == po.REASON_NO_K, (w, ext, ss, ds, p)
        else:
            assert p.ok, (w, ext, ss, ds, p)
            assert (p.P, p.k, p.shift, p.mask) == want, (w, ext, ss, ds, p, want)


def test_bruteforce_reproduces_the_worked_example():
    """The pages' region: fp32 (4, 32), strides (32, 1) -> (1, 4): P = 4, k = 2, shift 3, mask 3."""
    assert brute_plan(4, (4, 32), (32, 1), (1, 4)) == (4, 2, 3, 3)


def _disagreements(cases):
    bad = 0
    for w in (1, 4, 8, 16):
        for ext, ss, ds in cases:
            want = brute_plan(w, ext, ss, ds)
            p = po.plan(w, ext, ss, ds)
            bad += (None if not p.ok else (p.P, p.k, p.shift, p.mask)) != want
    return bad


def _shard_with(rule):
    def shard(extents, src, dst):
        e, s, d = po.drop_unit_modes(list(extents), list(src), list(dst))
        oe, os_, od = [e[0]], [s[0]], [d[0]]
        for i in range(1, len(e)):
            if rule(oe[-1], os_[-1], od[-1], e[i], s[i], d[i]):
                oe[-1] *= e[i]
                os_[-1], od[-1] = s[i], d[i]
            else:
                oe.append(e[i])
                os_.append(s[i])
                od.append(d[i])
        return oe, os_, od
    return shard


def _lane_offsets_half_mask(extent, strides, lanes, P, r, shift, mask, swz=None):
    return [po.swizzle_offset(swz, po.project(po.decompose(l + (r ^ ((l >> shift) & (mask >> 1))) * lanes, extent),
                                              strides)) for l in range(lanes)]


def _decompose_first_fastest(n, extent):
    out = []
    for e in extent:
        out.append(n % e)
        n //= e
    return out


PLANTED = {
    "shard merges where only the source merges": ("shard", _shard_with(lambda e0, s0, d0, e, s, d: s0 == e * s)),
    "shard merge rule transposed": ("shard", _shard_with(lambda e0, s0, d0, e, s, d: s0 * e0 == s and d0 * e0 == d)),
    "XOR key loses its top bit": ("lane_offsets", _lane_offsets_half_mask),
    "decompose runs the first axis fastest": ("decompose", _decompose_first_fastest),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_plan_oracle_mistake_disagrees(name, monkeypatch):
    attr, bad = PLANTED[name]
    monkeypatch.setattr(po, attr, bad)
    assert _disagreements(CASES[::3]) > 0


# ---------------------------------------------------------------------------
# The same cross-check on the measured gfx950 LDS geometry, against the
# library's half-wave planner (the program tpl_permute_staged runs: one
# 32-lane half of a wave, LDS reads through the source offsets, LDS writes
# through the destination offsets).  The measured model, restated: banks of
# 4 bytes; ds_read_b32 / ds_write_b32 (and sub-dword accesses) 32 banks in
# passes of 32 lanes; ds_read_b64 64 banks, 32 lanes; ds_write_b64 32 banks,
# 16 lanes; ds_read_b128 64 banks, 16 lanes of equal parity of lane bits
# 2..4; ds_write_b128 32 banks, 8 lanes.  Lanes asking one bank for the same
# dword do not conflict.

def measured_passes(w, is_write):
    lanes = np.arange(LANES)
    if w <= 4:
        return 32, [lanes]
    if w == 8:
        return (32, [lanes[i:i + 16] for i in range(0, 32, 16)]) if is_write else (64, [lanes])
    if is_write:
        return 32, [lanes[i:i + 8] for i in range(0, 32, 8)]
    parity = np.array([bin((l >> 2) & 7).count("1") & 1 for l in lanes])
    return 64, [lanes[parity == 0], lanes[parity == 1]]


def measured_step_ok(elem_offsets, w, is_write):
    nbanks, passes = measured_passes(w, is_write)
    dwords = max(1, w // 4)
    first = (elem_offsets * w) // 4
    for lanes in passes:
        holder = {}
        for l in lanes:
            for t in range(dwords):
                dw = int(first[l]) + t
                b = dw % nbanks
                if holder.setdefault(b, dw) != dw:
                    return False
    return True


def brute_plan_halfwave(w, ext, ss, ds):
    total = int(np.prod(ext))
    P = total // LANES
    lane = np.arange(LANES)
    for k in range(6):
        if (1 << k) > P or P % (1 << k):
            continue
        shift, mask = 5 - k, (1 << k) - 1
        if all(measured_step_ok(offsets(ext, ss, n), w, False) and measured_step_ok(offsets(ext, ds, n), w, True)
               for n in (lane + LANES * (r ^ ((lane >> shift) & mask)) for r in range(P))):
            return P, k, shift, mask
    return None


@pytest.mark.parametrize("w", [1, 2, 4, 8, 16])
def test_bruteforce_agrees_with_the_library_halfwave_plan(w):
    from tensor_layout_amd import tpl
    declined = found = 0
    for ext, ss, ds in CASES[::2]:
        want = brute_plan_halfwave(w, ext, ss, ds)
        p = tpl.tpl_plan(w, ext, ss, ds, geometry=tpl.TPL_GEOM_GFX950_HALFWAVE)
        if want is None:
            assert p.status == tpl.TPL_E_NO_K, (w, ext, ss, ds, p)
            declined += 1
        else:
            assert p.ok, (w, ext, ss, ds, p)
            assert (p.P, p.k, p.shift, p.mask) == want, (w, ext, ss, ds, p, want)
            found += 1
    assert found > 0


# The exhaustive 4-mode family: every shape of 4 modes with extents in
# {1, 2, 4, 8, 16, 32} and 32 to 256 elements (extent-1 modes included, so
# the oracle must drop them), row-major source, destination row-major in
# every one of the 24 axis orders.

def family4():
    import math
    vals = (1, 2, 4, 8, 16, 32)
    for ext in itertools.product(vals, repeat=4):
        if 32 <= math.prod(ext) <= 256:
            for order in itertools.permutations(range(4)):
                yield ext, row_major(ext, [0, 1, 2, 3], 0), row_major(ext, list(order), 0)


CASES4 = list(family4())


# Every layout at the 4-byte width; a third of them, a different third at each
# other width, so that every layout is also checked at a second width and the
# CPU suite stays short.
@pytest.mark.parametrize("w,start,step", [(4, 0, 1), (1, 0, 3), (2, 1, 3), (8, 2, 3), (16, 0, 3)])
def test_bruteforce_agrees_on_every_4_mode_layout(w, start, step):
    assert len(CASES4) == 8760
    for ext, ss, ds in CASES4[start::step]:
        want = brute_plan(w, ext, ss, ds)
        p = po.plan(w, ext, ss, ds)
        got = None if not p.ok else (p.P, p.k, p.shift, p.mask)
        assert got == want, (w, ext, ss, ds, p, want)
        if want is None:
            assert p.reason == po.REASON_NO_K
