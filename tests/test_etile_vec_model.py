"""CPU model of the element-tile kernel's vector form (plain operands, element
widths 1-4), run before the GPU does.  For small layouts it replays every
thread's accesses with the buffers placed at 256-byte aligned addresses (as
device allocations are), checks each global access and each LDS access, and
compares the result with the oracle's.  Written from the kernel's
description, not shared with it:

* tile TB x TA (TB along the destination-contiguous mode b, TA along the
  source-contiguous mode a), tiles in the tile kernel's order;
* loading: the source row piece of tile row bb starts lead(bb) = its address
  mod 16 bytes into a 16-byte aligned chunk; its chunks q with 16 q < lead +
  na w are read whole and written to LDS at vrow(bb) + 16 q, where vrow(bb) =
  bb rp + sk (bb >> le); thread t takes chunk t % QS of rows t / QS + i RS,
  then thread t < TB the extra chunk QS of row t / L + (TB / L) (t % L), L =
  128 / g being the lanes of one LDS write pass; in the first NS steps a
  lane whose row lies past the item or whose chunk lies past its row piece
  loads the tile's first chunk and writes it to its own slot, so that every
  lane writes in every step; no slot is written twice, and phase 2 reads
  none of those bytes;
* storing: tile column aa owns destination rows [delta, delta + TB) (from
  b0; clipped to the item), delta = the elements from its destination row's
  address at b0 to the next 16-byte boundary, so that its chunks are whole;
  the item's first tile also owns rows [0, delta), stored by thread aa of
  the extra step.  When some column has delta > 0 the tile loads TB + 16/w
  - 1 rows: the extra rows TB.. as one more step, thread f taking chunk f %
  (QS + 1) of row TB + f / (QS + 1).  A chunk inside the owned rows is
  stored whole, one it covers in part (the item's first or last rows)
  element by element; element (bb, aa) is read from LDS at vrow(bb) +
  lead(bb) + aa w.

The bank test replays one wave's LDS accesses on the measured gfx950 pass
structure and checks that no two lanes of a pass touch different dwords of
one bank."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl

NT = 256
ALIGN = 256
# w: (TB, TA, rp, sk, le, g)
VSHAPES = {1: (128, 128, 144, 16, 4, 16), 2: (128, 64, 152, 8, 3, 8), 4: (128, 32, 148, 4, 2, 4)}
# The tall tiles of 1- and 2-byte elements (twice the rows), which the
# planner takes for large launches.
TALL = {1: (256, 128, 152, 8, 4, 8), 2: (256, 64, 148, 4, 3, 4)}


def vrow(bb, rp, sk, le):
    return bb * rp + sk * (bb >> le)


def model(x, w, ext, ss, ds, offs, batch, item_strides=None, out=None, shape=None):
    """Replay the vector form on a 2-mode (plus batch) layout; buffers at
    ALIGN-aligned addresses, element offsets in offs.  Batch items lie one
    span apart unless item_strides = (source, destination) says otherwise;
    `out` (the destination buffer) may be given, else one of 0xCD bytes.
    `shape` (TB, TA, rp, sk, le, g) defaults to the width's tile."""
    TB, TA, rp, sk, le, g = shape or VSHAPES[w]
    QS, QD = TA * w // 16, TB * w // 16
    RS, CS = NT // QS, NT // QD
    a_mode = [i for i, s in enumerate(ss) if s == 1][0]
    b_mode = [i for i, d in enumerate(ds) if d == 1][0]
    e_a, e_b = ext[a_mode], ext[b_mode]
    s_b, d_a = ss[b_mode], ds[a_mode]
    span_s = 1 + sum((e - 1) * s for e, s in zip(ext, ss))
    span_d = 1 + sum((e - 1) * d for e, d in zip(ext, ds))
    istr_s, istr_d = item_strides if item_strides else (span_s, span_d)
    if out is None:
        out = np.full((offs[1] + (batch - 1) * istr_d + span_d) * w, 0xCD, dtype=np.uint8)
    xs = np.zeros(len(x) + 32, dtype=np.uint8)   # 16 bytes of slack on each side for chunk reads
    xs[16:16 + len(x)] = x
    chunks, stored = [], []
    E = 16 // w
    lds_bytes = vrow(TB + E - 1, rp, sk, le)
    ntb, nta = -(-e_b // TB), -(-e_a // TA)
    for item in range(batch):
        so, d_o = offs[0] + item * istr_s, offs[1] + item * istr_d
        for tile in range(ntb * nta):
            tbi, rest = tile % ntb, tile // ntb
            tq = rest % nta
            tai = (tq + tbi) % nta
            b0, a0 = tbi * TB, tai * TA
            nb, na = min(TB, e_b - b0), min(TA, e_a - a0)
            D0 = (d_o + a0 * d_a + b0) * w
            shifted = D0 % 16 != 0 or (d_a * w) % 16 != 0
            nl = min(TB + E - 1, e_b - b0) if shifted else nb   # rows loaded
            lds = np.full(lds_bytes, 0xEE, dtype=np.uint8)
            written = np.zeros(lds_bytes, dtype=bool)
            junk = np.zeros(lds_bytes, dtype=bool)   # slots written with bytes never read
            lead_s = {}
            # phase 1
            row0 = (so + b0 * s_b + a0) * w
            first = row0 - row0 % 16                         # the tile's first chunk
            for t in range(NT):
                main = [(t // QS + i * RS, t % QS) for i in range(TB // RS)]
                slots = list(main)
                if t < TB:
                    L = 128 // g
                    slots.append((t // L + (TB // L) * (t % L), QS))
                if shifted and t < (E - 1) * (QS + 1):
                    slots.append((TB + t // (QS + 1), t % (QS + 1)))
                for bb, q in slots:
                    row = (so + (b0 + bb) * s_b + a0) * w   # byte offset in the source buffer
                    lead = row % 16                          # buffer base is 16-byte aligned
                    if bb >= nl or q * 16 >= lead + na * w:
                        if (bb, q) in main:
                            # a main-step lane with nothing to load loads the
                            # tile's first chunk and writes it to its own slot
                            chunks.append(first)
                            l = vrow(bb, rp, sk, le) + 16 * q
                            assert 0 <= l and l + 16 <= vrow(bb + 1, rp, sk, le) and l + 16 <= lds_bytes
                            assert not written[l:l + 16].any() and not junk[l:l + 16].any()
                            junk[l:l + 16] = True
                        continue
                    lead_s[bb] = lead
                    A = row - lead + 16 * q
                    assert A % 16 == 0
                    # the chunk holds at least one byte of this row piece
                    assert A < row + na * w and A + 16 > row
                    chunks.append(A)
                    l = vrow(bb, rp, sk, le) + 16 * q
                    assert l % g == 0 and 0 <= l and l + 16 <= lds_bytes
                    assert l + 16 <= vrow(bb + 1, rp, sk, le)   # stays in its own row
                    assert not written[l:l + 16].any() and not junk[l:l + 16].any()
                    written[l:l + 16] = True
                    lds[l:l + 16] = xs[16 + A:16 + A + 16]
            # phase 2
            for t in range(NT):
                slots = [(t // QD + i * CS, t % QD) for i in range(TA // CS)]
                if t < TA:
                    slots.append((t, QD))
                for aa, q in slots:
                    if q < QD:
                        # the kernel reads the LDS bytes of every main-step
                        # slot before its stores, columns past the item
                        # included: rows outside [lo, hi) read row lo
                        Dx = (d_o + (a0 + aa) * d_a + b0) * w
                        dl = (16 - Dx % 16) % 16 if shifted else 0
                        lo_x = dl // w
                        hi_x = min(lo_x + TB, e_b - b0)
                        for j in range(16 // w):
                            bx = (dl + 16 * q) // w + j
                            bx = bx if lo_x <= bx < hi_x else lo_x
                            lx = vrow(bx, rp, sk, le) + (row0 + bx * s_b * w) % 16 + aa * w
                            assert 0 <= lx and lx + w <= min(lds_bytes, vrow(bx, rp, sk, le) + rp), (aa, q, bx)
                    if aa >= na:
                        continue
                    D = (d_o + (a0 + aa) * d_a + b0) * w
                    lead = D % 16
                    delta = ((16 - lead) % 16) // w
                    if q < QD:     # owned rows [delta, delta + TB), clipped to the item
                        rel, lo, hi = (16 - lead) % 16 + 16 * q, delta, min(delta + TB, e_b - b0)
                    else:          # the item's first rows [0, delta)
                        if tbi != 0 or lead == 0:
                            continue
                        rel, lo, hi = -lead, 0, min(delta, e_b - b0)
                    if rel >= hi * w:
                        continue
                    assert rel % w == 0 and hi <= nl
                    bbf = rel // w
                    full = rel >= lo * w and rel + 16 <= hi * w
                    # partial chunks only at the item's first or last rows
                    assert full or q == QD or hi == e_b - b0, (tile, aa, q)
                    for j in range(16 // w):
                        bb = bbf + j
                        if bb < lo or bb >= hi:
                            assert not full
                            continue
                        l = vrow(bb, rp, sk, le) + lead_s[bb] + aa * w
                        assert l % w == 0 and written[l:l + w].all()
                        e = D + bb * w
                        out[e:e + w] = lds[l:l + w]
                        stored.append(e // w)
                    if full:
                        assert (D + rel) % 16 == 0
    return out, chunks, stored


def footprint(ext, strides, batch, span, off):
    pts = {0}
    for e, s in zip(ext, strides):
        pts = {p + i * s for p in pts for i in range(e)}
    return {off + b * span + p for b in range(batch) for p in pts}


CASES = [
    # w, extents, src strides, dst strides, element offsets, batch
    (2, (150, 70), (73, 1), (1, 150), (0, 0), 1),        # odd pitch, ragged both ways
    (2, (300, 140), (141, 1), (1, 300), (3, 0), 1),      # several tiles, source offset
    (1, (140, 300), (301, 1), (1, 141), (5, 3), 1),      # odd pitches both sides, offsets
    (1, (260, 130), (133, 1), (1, 260), (0, 7), 2),      # unaligned destination start
    (4, (130, 40), (41, 1), (1, 133), (1, 0), 2),        # batch of two
    (4, (200, 90), (93, 1), (1, 203), (2, 1), 1),
    (2, (40, 20), (21, 1), (1, 40), (0, 0), 3),          # smaller than one tile
    (2, (16385, 9), (9, 1), (1, 16385), (0, 0), 1),      # destination pitch 16385: partial chunks
]


def _random_cases(n, seed):
    """Seeded small 2-D transposes with unaligned pitches or offsets on
    either side (the plan must take the vector form of the element tiles)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        w = int(rng.choice([1, 2, 4]))
        eb, ea = int(rng.integers(8, 300)), int(rng.integers(8, 300))
        ps = ea + int(rng.integers(0, 9))       # source row pitch (elements)
        pd = eb + int(rng.integers(0, 9))       # destination row pitch
        offs = (int(rng.integers(0, 8)), int(rng.integers(0, 8)))
        batch = int(rng.integers(1, 3))
        case = (w, (eb, ea), (ps, 1), (1, pd), offs, batch)
        p = tpl.tpl_plan(w, case[1], case[2], case[3], offs, batch)
        if p.ok and p.kernel == "etile":
            out.append(case)
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(24, 2024),
                         ids=lambda c: f"w{c[0]}_{c[1]}_{c[2][0]}_{c[3][1]}_{c[4]}_{c[5]}")
def test_etile_vector_model(case):
    w, ext, ss, ds, offs, batch = case
    p = tpl.tpl_plan(w, ext, ss, ds, offs, batch)
    assert p.ok and p.kernel == "etile", p
    TB, TA, rp, sk, le, g = VSHAPES[w]
    assert tuple(p.tile) == (TB, TA) and p.lds_pitch == rp
    span_s = 1 + sum((e - 1) * s for e, s in zip(ext, ss))
    span_d = 1 + sum((e - 1) * d for e, d in zip(ext, ds))
    x = synth.random_bytes(11, (offs[0] + batch * span_s) * w).copy()
    ref = np.full((offs[1] + batch * span_d) * w, 0xCD, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, offs, batch)
    out, chunks, stored = model(x, w, ext, ss, ds, offs, batch)
    fp_s = footprint(ext, ss, batch, span_s, offs[0])
    # every chunk read holds a byte of some source element of the layout
    for A in set(chunks):
        assert any((A + k) // w in fp_s for k in range(0, 16, w)), A
    # every element of the destination footprint is stored exactly once
    assert sorted(stored) == sorted(footprint(ext, ds, batch, span_d, offs[1]))
    assert np.array_equal(out, ref)


def _tall_cases(n, seed):
    """Seeded small 2-D transposes of 1- and 2-byte elements with unaligned
    pitches or offsets, replayed with the tall tiles (the planner takes them
    only for large launches, so the model runs them on small ones)."""
    rng = np.random.default_rng(seed)
    out = [(2, (300, 140), (141, 1), (1, 303), (0, 0), 1), (1, (600, 140), (141, 1), (1, 605), (3, 1), 1),
           (2, (260, 70), (73, 1), (1, 260), (0, 0), 2), (1, (257, 129), (131, 1), (1, 257), (0, 0), 1)]
    while len(out) < n:
        w = int(rng.choice([1, 2]))
        eb, ea = int(rng.integers(8, 700)), int(rng.integers(8, 300))
        ps = ea + int(rng.integers(0, 9))
        pd = eb + int(rng.integers(0, 9))
        offs = (int(rng.integers(0, 8)), int(rng.integers(0, 8)))
        if (ps * w) % 16 == 0 and (pd * w) % 16 == 0 and (offs[0] * w) % 16 == 0 and (offs[1] * w) % 16 == 0:
            continue
        out.append((w, (eb, ea), (ps, 1), (1, pd), offs, int(rng.integers(1, 3))))
    return out


@pytest.mark.parametrize("case", _tall_cases(20, 4096),
                         ids=lambda c: f"w{c[0]}_{c[1]}_{c[2][0]}_{c[3][1]}_{c[4]}_{c[5]}")
def test_etile_tall_model(case):
    w, ext, ss, ds, offs, batch = case
    span_s = 1 + sum((e - 1) * s for e, s in zip(ext, ss))
    span_d = 1 + sum((e - 1) * d for e, d in zip(ext, ds))
    x = synth.random_bytes(12, (offs[0] + batch * span_s) * w).copy()
    ref = np.full((offs[1] + batch * span_d) * w, 0xCD, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, offs, batch)
    out, chunks, stored = model(x, w, ext, ss, ds, offs, batch, shape=TALL[w])
    fp_s = footprint(ext, ss, batch, span_s, offs[0])
    for A in set(chunks):
        assert any((A + k) // w in fp_s for k in range(0, 16, w)), A
    assert sorted(stored) == sorted(footprint(ext, ds, batch, span_d, offs[1]))
    assert np.array_equal(out, ref)


def test_etile_tall_planner_choice():
    """The planner's rule: tall tiles for unaligned destination rows from 2048
    tall tiles, for bf16 with aligned destination rows from 16384; the plan
    reports the tall tile's placement."""
    cases = [
        # w, extents, src strides, dst strides, tall
        (2, (8192, 8192), (8192, 1), (1, 8193), True),
        (2, (4096, 4096), (4096, 1), (1, 4097), False),     # 1024 tall tiles
        (1, (8192, 8192), (8192, 1), (1, 8195), True),      # 2048
        (1, (4096, 8192), (8192, 1), (1, 4099), False),     # 1024
        (2, (16384, 16384), (16385, 1), (1, 16384), True),  # aligned destination, 16384
        (2, (8192, 8192), (8196, 1), (1, 8192), False),     # aligned destination, 4096
        (1, (16384, 16384), (16387, 1), (1, 16384), False),  # u8 with aligned destination rows
        (4, (8192, 8192), (8192, 1), (1, 8193), False),     # no tall 4-byte tile
        (2, (8000, 8100), (8100, 1), (1, 8003), True),      # ragged both ways
    ]
    for w, ext, ss, ds, tall in cases:
        p = tpl.tpl_plan(w, ext, ss, ds)
        assert p.ok and p.kernel == "etile", (ext, p)
        TB, TA, rp, sk, le, g = TALL[w] if tall else VSHAPES[w]
        assert tuple(p.tile) == (TB, TA) and p.lds_pitch == rp, (w, ext, ss, ds, p)


def ways(addrs, width, nbanks):
    used = {}
    for a in addrs:
        for dw in range(a // 4, (a + max(width, 4) - 1) // 4 + 1):
            used.setdefault(dw % nbanks, set()).add(dw)
    return max(len(s) for s in used.values())


def ways_aligned(addrs, width, nbanks):
    """ways() for accesses aligned to their width: an element of 1 or 2
    bytes then lies in one dword (ways() counts the 4 bytes from its
    address, which may reach into the next dword)."""
    used = {}
    for a in addrs:
        assert a % width == 0
        for dw in range(a // 4, (a + width - 1) // 4 + 1):
            used.setdefault(dw % nbanks, set()).add(dw)
    return max(len(s) for s in used.values())


def check_banks(w, shape, pm, read_ways):
    """Measured gfx950 passes: b128 writes 8 lanes, b64 writes 16 lanes (32
    banks), b32 writes and reads of up to 4 bytes 32 lanes (32 banks); lanes
    on one dword share it.  pm: the change of a source row's lead per row
    (the source row pitch in bytes mod 16); the destination is aligned.
    read_ways counts the element reads of phase 2."""
    TB, TA, rp, sk, le, g = shape
    QS, QD = TA * w // 16, TB * w // 16
    for L0 in sorted({0, (3 * w) % 16}):
        lead = lambda bb: (L0 + bb * pm) % 16
        # phase 1: one wave's chunk writes (slot s = lane + 64 i: row s // QS, chunk s % QS)
        for i in range(TB * QS // 64):
            slots = [((s // QS), s % QS) for s in range(64 * i, 64 * i + 64)]
            if g == 16:
                passes = [[vrow(bb, rp, sk, le) + 16 * q for bb, q in slots[p:p + 8]] for p in range(0, 64, 8)]
                width = 16
            elif g == 8:
                passes = [[vrow(bb, rp, sk, le) + 16 * q + 8 * (((q >> 3) & 1) ^ part) for bb, q in slots[p:p + 16]]
                          for part in (0, 1) for p in range(0, 64, 16)]
                width = 8
            else:
                passes = [[vrow(bb, rp, sk, le) + 16 * q + part for bb, q in slots[p:p + 32]]
                          for part in (0, 4, 8, 12) for p in range(0, 64, 32)]
                width = 4
            for ps in passes:
                assert ways(ps, width, 32) == 1, (w, i, ps)
        # phase 1, the extra chunk of each row: lane t of the first TB takes row
        # t / L + (TB / L) (t % L), L = 128 / g lanes per write pass
        L = 128 // g
        rows = [t // L + (TB // L) * (t % L) for t in range(TB)]
        assert sorted(rows) == list(range(TB))
        for p0 in range(0, TB, L):
            pr = rows[p0:p0 + L]
            if g == 16:
                passes = [[vrow(bb, rp, sk, le) + 16 * QS for bb in pr]]
            elif g == 8:   # chunk QS: (QS >> 3) & 1 picks the half written first
                h = (QS >> 3) & 1
                passes = [[vrow(bb, rp, sk, le) + 16 * QS + 8 * (h ^ part) for bb in pr] for part in (0, 1)]
            else:
                passes = [[vrow(bb, rp, sk, le) + 16 * QS + part for bb in pr] for part in (0, 4, 8, 12)]
            for ps in passes:
                assert ways(ps, g, 32) == 1, (w, "extra", p0)
        # phase 2: element j of one wave's chunks (lane -> chunk lane % QD of column lane // QD)
        for c0 in range(0, TA, max(1, 64 // QD)):
            for j in range(16 // w):
                for first in (0, 32):
                    addrs = []
                    for lane in range(first, first + 32):
                        q, aa = lane % QD, c0 + lane // QD
                        bb = q * (16 // w) + j
                        if aa < TA and bb < TB:
                            addrs.append(vrow(bb, rp, sk, le) + lead(bb) + aa * w)
                    assert read_ways(addrs, w, 32) == 1, (w, pm, L0, c0, j, first)


@pytest.mark.parametrize("w", [1, 2, 4])
@pytest.mark.parametrize("pm", [0, 2, 8, 14])
def test_etile_vector_lds_is_conflict_free(w, pm):
    if pm % w:
        pytest.skip("leads are multiples of the element width")
    check_banks(w, VSHAPES[w], pm, ways)


def shifted_phase2_ways(w, shape):
    """Phase 2 with unaligned destination rows: column aa's destination lead
    is (D0 + aa * dpm) mod 16 (dpm: the destination row pitch in bytes mod
    16), so its chunk q starts at row delta / w + q * E (delta the bytes to
    the next 16-byte boundary) and step j reads that row + j.  Returns the
    worst and the mean number of dwords per bank over one half-wave's
    reads, across leads."""
    TB, TA, rp, sk, le, g = shape
    QD, E = TB * w // 16, 16 // w
    worst, tot, n = 1, 0, 0
    for pm in sorted({0, 2 * w % 16, 8}):
        for dpm in range(w, 16, w):
            for L0 in sorted({0, (3 * w) % 16}):
                for D0 in (0, (5 * w) % 16):
                    for c0 in range(0, TA, max(1, 64 // QD)):
                        for j in range(E):
                            for first in (0, 32):
                                addrs = []
                                for lane in range(first, first + 32):
                                    q, aa = lane % QD, c0 + lane // QD
                                    lead = (D0 + aa * dpm) % 16
                                    bb = ((16 - lead) % 16) // w + q * E + j
                                    addrs.append(vrow(bb, rp, sk, le) + (L0 + bb * pm) % 16 + aa * w)
                                k = ways_aligned(addrs, w, 32)
                                worst, tot, n = max(worst, k), tot + k, n + 1
    return worst, tot / n


def test_etile_shifted_form_banks():
    """Unaligned destination rows give each column of a half-wave its own
    first row.  The tall bf16 tile reads one column per half-wave and stays
    conflict-free; the tiles with several columns per half-wave do not
    (rocprofv3 on MI355X: 0.01, 0.40, 0.70 and 0.45 conflict cycles per
    active LDS cycle for tall bf16, bf16, u8 and tall u8)."""
    assert shifted_phase2_ways(2, TALL[2]) == (1, 1.0)
    for w, shape, mean_max in ((2, VSHAPES[2], 1.6), (1, VSHAPES[1], 2.7), (1, TALL[1], 1.7)):
        worst, mean = shifted_phase2_ways(w, shape)
        assert 1 < mean < mean_max, (w, shape, worst, mean)


@pytest.mark.parametrize("w", [1, 2])
def test_etile_tall_lds_is_conflict_free(w):
    """The tall tiles over every lead step: phase 1 on the same pass model;
    phase 2 has 32 rows of one column per half-wave (bf16) or 16 rows of two
    (bytes), so element reads are counted by the dword that holds them."""
    for pm in range(0, 16, w):
        check_banks(w, TALL[w], pm, ways_aligned)


def test_etile_vector_shapes_match_the_library():
    """The placement constants the model uses are the ones the planner
    reports; 8-byte elements keep the element form (row + one element)."""
    for w, (TB, TA, rp, sk, le, g) in VSHAPES.items():
        p = tpl.tpl_plan(w, (500, 300), (301, 1), (1, 500))
        assert p.kernel == "etile" and tuple(p.tile) == (TB, TA) and p.lds_pitch == rp and p.P == 16 // w, (w, p)
    p = tpl.tpl_plan(8, (500, 300), (301, 1), (1, 500))
    assert p.kernel == "etile" and tuple(p.tile) == (64, 32) and p.lds_pitch == 32 * 8 + 8 and p.P == 1, p


def test_etile_vector_lead_sweep_is_conflict_free():
    """Phase 2 over every tile lead L0 and every per-row lead step pm (the
    source pitch in bytes mod 16), aligned destination; the tall tiles with
    element reads counted by the dword that holds them."""
    shapes = [(w, sh, ways) for w, sh in VSHAPES.items()] + [(w, sh, ways_aligned) for w, sh in TALL.items()]
    for w, (TB, TA, rp, sk, le, g), count in shapes:
        QD = TB * w // 16
        for pm in range(0, 16, w):
            for L0 in range(0, 16, w):
                for c0 in range(0, TA, max(1, 64 // QD)):
                    for j in range(16 // w):
                        for first in (0, 32):
                            addrs = []
                            for lane in range(first, first + 32):
                                q, aa = lane % QD, c0 + lane // QD
                                bb = q * (16 // w) + j
                                addrs.append(vrow(bb, rp, sk, le) + (L0 + bb * pm) % 16 + aa * w)
                            assert count(addrs, w, 32) == 1, (w, TB, pm, L0, c0, j, first)


@pytest.mark.parametrize("w,n,pitch,batch,gap,offset", [(1, 100, 101, 7, 0, 0), (2, 60, 61, 9, 3, 1), (4, 30, 33, 4, 5, 2)])
def test_etile_vector_model_in_place(w, n, pitch, batch, gap, offset):
    """Square transposes in place, one tile per item, items n pitch + gap
    elements apart: every chunk an item reads is read before any of the
    item is written (one workgroup per item), and the buffer ends as the
    oracle's permutation written over the input (padding and gaps kept)."""
    item = n * pitch + gap
    ext, ss, ds = (batch, n, n), (item, pitch, 1), (item, 1, pitch)
    p = tpl.tpl_plan(w, ext, ss, ds, (offset, offset), 1, geometry=tpl.TPL_GEOM_GFX950_INPLACE)
    assert p.ok and p.kernel == "etile", p
    x = synth.random_bytes(13, (offset + batch * item) * w).copy()
    ref = x.copy()
    oracle.permute(x, ref, w, ext, ss, ds, (offset, offset), 1)
    # the model reads the input as it was: each item is one tile, loaded
    # whole before its stores, and items never write bytes of other items
    out, _, _ = model(x, w, (n, n), (pitch, 1), (1, pitch), (offset, offset), batch, (item, item), out=x.copy())
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("w,n,pitch,batch,gap,offset", [(1, 100, 101, 7, 0, 0), (2, 60, 61, 9, 3, 1), (1, 128, 131, 3, 5, 2)])
def test_etile_tall_model_in_place(w, n, pitch, batch, gap, offset):
    """The same in-place property with the tall tiles (the planner takes them
    for such layouts from 2048 items): one tile per item, read whole before
    its stores, the buffer ends as the oracle's permutation."""
    item = n * pitch + gap
    ext, ss, ds = (batch, n, n), (item, pitch, 1), (item, 1, pitch)
    x = synth.random_bytes(14, (offset + batch * item) * w).copy()
    ref = x.copy()
    oracle.permute(x, ref, w, ext, ss, ds, (offset, offset), 1)
    out, _, _ = model(x, w, (n, n), (pitch, 1), (1, pitch), (offset, offset), batch, (item, item), out=x.copy(),
                      shape=TALL[w])
    assert np.array_equal(out, ref)
