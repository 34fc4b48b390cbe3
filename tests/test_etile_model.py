"""CPU model of the element-tile kernel's element form (k_etile on swizzled
operands; plain operands take the vector form, modelled in
test_etile_vec_model.py), run before the GPU does: for small layouts it
replays every thread's accesses of both phases on numpy buffers (the
swizzle is an address map on top, covered by the GPU parity tests), checks each global access against the
layout's footprint and each LDS access against the tile, and compares the
result with the oracle's.  Written from the kernel's description (tiles of
TB x TA elements in the tile kernel's order, LDS rows of TA elements plus
one unit of max(w, 4) bytes, thread t on column t % TA stepping 256 / TA
rows while loading, on column t % TB stepping 256 / TB rows while
storing; a lane outside the item loads the tile's first element and
writes it to its own LDS slot, so that every lane writes in every step),
not shared with it."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl

NT = 256
SHAPES = {1: (128, 128), 2: (128, 64), 4: (128, 32), 8: (64, 32), 16: (64, 16)}


def model(x, w, ext, ss, ds, offs, batch, plan_tile, pitch):
    """Replay k_etile on the shard of a 2-mode (plus batch) layout."""
    TB, TA = plan_tile
    a_mode = [i for i, s in enumerate(ss) if s == 1][0]
    b_mode = [i for i, d in enumerate(ds) if d == 1][0]
    e_a, e_b = ext[a_mode], ext[b_mode]
    s_b, d_a = ss[b_mode], ds[a_mode]
    span_s = 1 + sum((e - 1) * s for e, s in zip(ext, ss))
    span_d = 1 + sum((e - 1) * d for e, d in zip(ext, ds))
    out = np.zeros((offs[1] + batch * span_d) * w, dtype=np.uint8)
    touched_s, touched_d = set(), set()
    ntb, nta = -(-e_b // TB), -(-e_a // TA)
    RA, RB = NT // TA, NT // TB
    for item in range(batch):
        so, d_o = offs[0] + item * span_s, offs[1] + item * span_d
        for tile in range(ntb * nta):
            tbi, rest = tile % ntb, tile // ntb
            tq = rest % nta
            tai = (tq + tbi) % nta
            b0, a0 = tbi * TB, tai * TA
            nb, na = min(TB, e_b - b0), min(TA, e_a - a0)
            lds = np.full(TB * pitch, 0xEE, dtype=np.uint8)
            real = np.zeros(TB * pitch, dtype=bool)
            junk = np.zeros(TB * pitch, dtype=bool)
            first = so + b0 * s_b + a0                    # the tile's first element
            for t in range(NT):
                aa, bb1 = t % TA, t // TA
                for i in range(TB // RA):
                    bb = bb1 + i * RA
                    l = bb * pitch + aa * w
                    assert 0 <= l and l + w <= TB * pitch
                    assert not real[l:l + w].any() and not junk[l:l + w].any()   # one writer per slot
                    if aa < na and bb < nb:
                        e = so + (b0 + bb) * s_b + a0 + aa
                        real[l:l + w] = True
                    else:
                        # every lane writes in every step: one outside the item
                        # loads the tile's first element into its own slot
                        e = first
                        junk[l:l + w] = True
                    touched_s.add(e)
                    lds[l:l + w] = x[e * w:(e + 1) * w]
            for t in range(NT):
                bb, aa2 = t % TB, t // TB
                for i in range(TA // RB):
                    aa = aa2 + i * RB
                    l = bb * pitch + aa * w
                    assert 0 <= l and l + w <= TB * pitch   # every lane reads, in bounds
                    if bb < nb and aa < na:
                        assert real[l:l + w].all()
                        e = d_o + (a0 + aa) * d_a + b0 + bb
                        touched_d.add(e)
                        l = bb * pitch + aa * w
                        out[e * w:(e + 1) * w] = lds[l:l + w]
    return out, touched_s, touched_d


def footprint(ext, strides, batch, span, off):
    pts = {0}
    for e, s in zip(ext, strides):
        pts = {p + i * s for p in pts for i in range(e)}
    return {off + b * span + p for b in range(batch) for p in pts}


CASES = [
    # w, extents, src strides, dst strides, element offsets, batch
    (2, (150, 70), (73, 1), (1, 150), (0, 0), 1),        # odd pitch, ragged both ways
    (1, (140, 130), (131, 1), (1, 141), (5, 3), 1),      # odd pitches both sides, offsets
    (4, (130, 40), (41, 1), (1, 133), (1, 0), 2),        # batch of two
    (8, (70, 33), (35, 1), (1, 70), (0, 2), 1),
    (2, (40, 20), (21, 1), (1, 40), (0, 0), 3),          # smaller than one tile
]


def _random_cases(n, seed):
    """Seeded small 2-D transposes that plan as element tiles: 8-byte
    elements with unaligned pitches (the element form runs them), and 1- to
    4-byte ones (the element form runs those when an operand is swizzled;
    the model here replays the same tiles without the swizzle map)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        w = int(rng.choice([1, 2, 4, 8, 8]))
        eb, ea = int(rng.integers(8, 200)), int(rng.integers(8, 200))
        ps = ea + int(rng.integers(0, 5))
        pd = eb + int(rng.integers(0, 5))
        offs = (int(rng.integers(0, 4)), int(rng.integers(0, 4)))
        batch = int(rng.integers(1, 3))
        case = (w, (eb, ea), (ps, 1), (1, pd), offs, batch)
        p = tpl.tpl_plan(w, case[1], case[2], case[3], offs, batch)
        if p.ok and p.kernel == "etile":
            out.append(case)
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(16, 77),
                         ids=lambda c: f"w{c[0]}_{c[1]}_{c[2][0]}_{c[3][1]}_{c[4]}_{c[5]}")
def test_etile_model(case):
    w, ext, ss, ds, offs, batch = case
    p = tpl.tpl_plan(w, ext, ss, ds, offs, batch)
    assert p.ok and p.kernel == "etile", p
    assert tuple(p.tile) == SHAPES[w]
    span_s = 1 + sum((e - 1) * s for e, s in zip(ext, ss))
    span_d = 1 + sum((e - 1) * d for e, d in zip(ext, ds))
    x = synth.random_bytes(9, (offs[0] + batch * span_s) * w).copy()
    ref = np.zeros((offs[1] + batch * span_d) * w, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, offs, batch)
    TB, TA = p.tile
    out, ts, td = model(x, w, ext, ss, ds, offs, batch, p.tile, TA * w + max(w, 4))
    assert ts <= footprint(ext, ss, batch, span_s, offs[0])
    assert td == footprint(ext, ds, batch, span_d, offs[1])
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("w", [1, 2, 4, 8, 16])
def test_etile_column_reads_hit_distinct_banks(w):
    """Phase 2: the lanes of one pass read one element each from neighbouring
    LDS rows (row pitch = TA w + max(w, 4) bytes).  Every lane's dwords lie in
    banks no other lane of its pass uses (32 lanes per pass up to 8-byte
    elements -- 64 banks for 8-byte reads -- and 16 for 16-byte ones)."""
    TB, TA = SHAPES[w]
    pitch = TA * w + max(w, 4)
    lanes = 16 if w == 16 else 32
    banks = 64 if w >= 8 else 32
    for aa in (0, 1, TA - 1):
        for first in (0, lanes):
            used = {}
            for lane in range(lanes):
                byte = (first + lane) * pitch + aa * w
                for dw in range(byte // 4, (byte + max(w, 4) - 1) // 4 + 1 if w >= 4 else byte // 4 + 1):
                    b = dw % banks
                    assert used.get(b, dw) == dw, (w, aa, lane)
                    used[b] = dw


@pytest.mark.parametrize("w", [1, 2, 4, 8])
def test_etile_swizzled_plans_take_the_element_form(w):
    """A swizzle granule under 16 bytes (2^base elements) rules out 16-byte
    chunks: the plan reports the element form's pitch (row + max(w, 4)).
    (A 16-byte element's granule is never under 16 bytes.)"""
    base = 0 if w >= 8 else 1
    p = tpl.tpl_plan(w, (150, 70), (73, 1), (1, 150), dst_swizzle=(1, base, 3))
    assert p.ok and p.kernel == "etile", p
    TB, TA = SHAPES[w]
    assert tuple(p.tile) == (TB, TA) and p.lds_pitch == TA * w + max(w, 4) and p.P == 1
