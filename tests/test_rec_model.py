"""CPU model of the records kernel's index arithmetic (k_rec), run before the
GPU does: for small layouts it replays every thread's accesses of both
phases on numpy buffers, checks that each one stays inside the layout's
footprint, and that the result equals the oracle's.  The model is written
from the kernel's description (tile of TR records, LDS in record order --
for fields to records with elements of 4 bytes or more, each 16-byte chunk
turned by whole dwords or halves -- dense block on one side, 16-byte pieces
of field rows on the other, element by element for a short last tile), not
shared with it.  LDS is a byte array here, so a chunk turned one way on the
chunk side and read another way on the piece side shows up as a wrong
result."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl

NT = 256


def turn_dwords(w, c, turned=True):
    """Dword positions chunk c of a full tile is turned by in LDS."""
    if not turned:
        return 0
    if w <= 4:
        return (c // 8) % 4
    if w == 8:
        return 2 * ((c // 16) % 2)
    return 0


def chunk_into_lds(lds, c, data, w, turned):
    r = turn_dwords(w, c, turned)
    for j in range(4):
        pos = (j + r) % 4
        lds[c * 16 + pos * 4:c * 16 + pos * 4 + 4] = data[j * 4:j * 4 + 4]


def chunk_from_lds(lds, c, w, turned):
    r = turn_dwords(w, c, turned)
    out = np.zeros(16, dtype=np.uint8)
    for j in range(4):
        pos = (j + r) % 4
        out[j * 4:j * 4 + 4] = lds[c * 16 + pos * 4:c * 16 + pos * 4 + 4]
    return out


def elem_slot(b, w, turned=True):
    """LDS byte of element byte b of a full tile's dense block."""
    c, off = divmod(b, 16)
    return c * 16 + (off + 4 * turn_dwords(w, c, turned)) % 16


def model(x, w, ext, ss, ds, batch, dense_src, F, TR, nrec, fstride, batch_offsets):
    """Replay k_rec; returns (output bytes, set of source and destination element offsets touched)."""
    out = np.zeros(batch_offsets["dst_size"] * w, dtype=np.uint8)
    touched_s, touched_d = set(), set()
    ce = 16 // w
    turned = not dense_src and w >= 4
    ntr = -(-nrec // TR)
    for item, (so, d_o) in enumerate(batch_offsets["items"]):
        for ti in range(ntr):
            r0 = ti * TR
            nr = min(TR, nrec - r0)
            lds = np.full(TR * F * w, 0xEE, dtype=np.uint8)
            block = so + r0 * F if dense_src else d_o + r0 * F
            rows = d_o + r0 if dense_src else so + r0
            if nr == TR:
                nq = TR // ce
                nchunks = F * TR // ce
                # phase 1
                if dense_src:
                    for c in range(nchunks):
                        e0 = block + c * ce
                        touched_s.update(range(e0, e0 + ce))
                        chunk_into_lds(lds, c, x[e0 * w:(e0 + ce) * w], w, turned)
                else:
                    for g in range(nchunks):
                        q, f = g % nq, g // nq
                        for k in range(ce):
                            e = rows + f * fstride + q * ce + k
                            touched_s.add(e)
                            sl = elem_slot(((q * ce + k) * F + f) * w, w, turned)
                            lds[sl:sl + w] = x[e * w:(e + 1) * w]
                # phase 2
                if dense_src:
                    for g in range(nchunks):
                        q, f = g % nq, g // nq
                        for k in range(ce):
                            e = rows + f * fstride + q * ce + k
                            touched_d.add(e)
                            sl = elem_slot(((q * ce + k) * F + f) * w, w, turned)
                            out[e * w:(e + 1) * w] = lds[sl:sl + w]
                else:
                    for c in range(nchunks):
                        e0 = block + c * ce
                        touched_d.update(range(e0, e0 + ce))
                        out[e0 * w:(e0 + ce) * w] = chunk_from_lds(lds, c, w, turned)
            else:
                for i in range(nr * F):
                    f, r = i // nr, i % nr
                    e = block + r * F + f if dense_src else rows + f * fstride + r
                    touched_s.add(e)
                    lds[(r * F + f) * w:(r * F + f + 1) * w] = x[e * w:(e + 1) * w]
                for i in range(nr * F):
                    f, r = i // nr, i % nr
                    e = rows + f * fstride + r if dense_src else block + r * F + f
                    touched_d.add(e)
                    out[e * w:(e + 1) * w] = lds[(r * F + f) * w:(r * F + f + 1) * w]
    return out, touched_s, touched_d


def footprint(ext, strides, batch, span):
    pts = {0}
    for e, s in zip(ext, strides):
        pts = {p + i * s for p in pts for i in range(e)}
    return {b * span + p for b in range(batch) for p in pts}


CASES = [
    # w, extents, src strides, dst strides, batch
    (4, (600, 3), (3, 1), (1, 600), 2),        # float3 records -> fields, a short last tile
    (4, (3, 600), (600, 1), (1, 3), 2),        # and back
    (1, (5000, 3), (3, 1), (1, 5008), 1),      # RGB -> planes (rows padded to 16 bytes)
    (1, (3, 5000), (5008, 1), (1, 3), 1),      # planes -> RGB
    (4, (200, 17), (17, 1), (1, 208), 1),      # 17-float records
    (2, (1000, 6), (6, 1), (1, 1000), 3),
    (8, (300, 3), (3, 1), (1, 300), 1),
    (4, (5, 2), (2, 1), (1, 8), 1),            # one full tile of 4 records, one of 1
    (2, (3, 2000), (2000, 1), (1, 3), 2),      # fp16 planes -> 3-field records
    (8, (3, 700), (700, 1), (1, 3), 1),        # 8-byte fields to records: chunks turned by halves
    (4, (5, 900), (900, 1), (1, 5), 1),        # fp32 fields to records: chunks turned by dwords
    (1, (6, 4000), (4000, 1), (1, 6), 1),      # even field count
]


def test_turn_is_a_permutation_of_each_chunk():
    for w in (1, 2, 4, 8, 16):
        for c in range(64):
            assert sorted(elem_slot(c * 16 + o, w) - c * 16 for o in range(0, 16, 4)) == [0, 4, 8, 12]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"w{c[0]}_{c[1]}")
def test_records_kernel_model(case):
    w, ext, ss, ds, batch = case
    p = tpl.tpl_plan(w, ext, ss, ds, batch=batch)
    assert p.ok and p.kernel == "rec", p
    src_records = ext[1] <= ext[0]
    F = ext[1] if src_records else ext[0]
    nrec = ext[0] if src_records else ext[1]
    TR = p.tile[0] if src_records else p.tile[1]
    fstride = ds[1] if src_records else ss[0]
    assert TR % (16 // w) == 0 and TR <= nrec
    span_s = 1 + sum((e - 1) * s for e, s in zip(ext, ss))
    span_d = 1 + sum((e - 1) * s for e, s in zip(ext, ds))
    x = synth.random_bytes(7, batch * span_s * w).copy()
    ref = np.zeros(batch * span_d * w, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, (0, 0), batch)
    offs = {"items": [(b * span_s, b * span_d) for b in range(batch)], "dst_size": batch * span_d}
    out, ts, td = model(x, w, ext, ss, ds, batch, src_records, F, TR, nrec, fstride, offs)
    assert ts <= footprint(ext, ss, batch, span_s)
    assert td == footprint(ext, ds, batch, span_d)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("w", [1, 2, 4, 8])
@pytest.mark.parametrize("F", [3, 5, 7, 17])
def test_turn_spreads_piece_lanes_over_all_banks(w, F):
    """Turned layout, piece phase, odd F: the 32 lanes of one LDS pass (consecutive q, same k
    and f) touch 32 different banks -- 4-byte banks, 32 per 128 bytes for
    accesses of up to a dword, 64 per 256 bytes for 8-byte ones.  In plain
    record order they would share 8 (4-way conflicts)."""
    ce = 16 // w
    nbanks = 32 if w <= 4 else 64
    for k in range(ce):
        for f in range(F):
            for q0 in (0, 32, 64):
                banks = [elem_slot(((q * ce + k) * F + f) * w, w) // 4 % nbanks for q in range(q0, q0 + 32)]
                if w == 8:
                    assert len(set(banks)) == 32 and all(b % 2 == banks[0] % 2 for b in banks)
                else:
                    assert len(set(banks)) == 32
                plain = [((q * ce + k) * F + f) * w // 4 % nbanks for q in range(q0, q0 + 32)]
                assert len(set(plain)) <= 16


@pytest.mark.parametrize("F", [1, 3, 5, 7, 9, 17])
def test_fp32_field_reads_in_lane_order_hit_distinct_banks(F):
    """Records to fields with 4-byte fields and odd F: lane t of the piece
    phase reads its piece's records q*4 + (k ^ x) at step k, x = (t >> 3) & 3.
    The 32 lanes of one read pass (consecutive q, same f and k) touch 32
    distinct banks (4-byte banks, 32 per pass); in plain record order
    (x = 0) only 8.  The order is a permutation of each piece's records."""
    for f in range(F):
        for k in range(4):
            for q0 in (0, 32, 96):
                lanes = range(q0, q0 + 32)
                banks = [((q * 4 + (k ^ ((q >> 3) & 3))) * F + f) % 32 for q in lanes]
                assert len(set(banks)) == 32, (F, f, k, q0)
                plain = [((q * 4 + k) * F + f) % 32 for q in lanes]
                assert len(set(plain)) == 8
    for x in range(4):
        assert sorted(k ^ x for k in range(4)) == [0, 1, 2, 3]
