"""Pins of the plan oracle (canonicalise, regroup, P, XOR-k search) in the pages' geometry.

What pins it, besides itself:
* the worked example's printed IR: the per-lane program's read and write
  indices at (shift 3, mask 3) must equal the printed expressions, and the
  search must land on P = 4, shift 3, mask 3;
* the "How inputs change the algorithm" table: 4-byte P x 32 transposes admit
  a k, k = 0 means no swizzle, stride-1 sub-4-byte reads can decline;
* closed forms of the bank pattern of the worked example at k = 0, 1, 2;
* the result is independent of k (the XOR reorders accesses, never values).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import plan_oracle as po
from tensor_layout_amd import synth
from tests import goldens


def sf_region_plan():
    g = goldens.sf_ir()
    return po.plan(4, g["region_extents"], g["src_strides"], g["dst_strides"])


def pin_worked_example_plan() -> bool:
    g = goldens.sf_ir()
    p = sf_region_plan()
    return (p.ok and p.extent == [4, 32] and p.src_str == [32, 1] and p.dst_str == [1, 4]
            and p.P == g["P"] and p.shift == g["shift"] and p.mask == g["mask"])


def pin_lane_program_matches_ir() -> bool:
    """Per-lane offsets at (shift 3, mask 3) equal the printed IR (stage 0)."""
    g = goldens.sf_ir()
    ext, ss, ds = [4, 32], [32, 1], [1, 4]
    for r in range(4):
        rd = po.lane_offsets(ext, ss, 32, 4, r, g["shift"], g["mask"])
        wr = po.lane_offsets(ext, ds, 32, 4, r, g["shift"], g["mask"])
        for tx in range(32):
            if rd[tx] != goldens.eval_index(g["read"], s=0, r=r, tx=tx):
                return False
            if wr[tx] != goldens.eval_index(g["write"], s=0, r=r, tx=tx):
                return False
    return True


def pin_four_byte_family() -> bool:
    """P x 32 <-> 32 x P fp32 transposes: a k exists, and it is log2 P.

    Closed form: the write offsets are j + P*lane, so lanes lane and
    lane + 32/P land in one bank unless their keys differ; 32 lanes need P
    distinct keys in every bank class, i.e. k = log2 P bits of the lane id.
    """
    for k in range(6):
        P = 1 << k
        p = po.plan(4, (P, 32), (32, 1), (1, P))
        if not (p.ok and p.P == P and p.k == k and p.mask == P - 1 and p.shift == 5 - k):
            return False
    return True


def pin_sub_word_declines() -> bool:
    """Stride-1 reads of 1- and 2-byte elements put two lanes in one bank: decline."""
    for w in (1, 2):
        if po.plan(w, (4, 32), (32, 1), (1, 4)).reason != po.REASON_NO_K:
            return False
    return po.plan(2, (128,), (1,), (1,)).reason == po.REASON_NO_K


def pin_identity_k0() -> bool:
    """A plain 32-element fp32 copy is conflict-free unswizzled: k = 0, mask 0."""
    p = po.plan(4, (32,), (1,), (1,))
    return p.ok and p.P == 1 and p.k == 0 and p.mask == 0


PINS = [pin_worked_example_plan, pin_lane_program_matches_ir, pin_four_byte_family,
        pin_sub_word_declines, pin_identity_k0]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_plan_oracle_pin(pin):
    assert pin()


def test_worked_example_bank_closed_forms():
    """Write phase of the worked example, r = 0: bank = (4*lane + j) mod 32.

    k = 0: lanes lane, lane+8, lane+16, lane+24 share a bank (4-way);
    k = 1 (shift 4): lanes tx and tx+8 still collide;
    k = 2 (shift 3): every bank is hit exactly once.
    """
    ext, ds = [4, 32], [1, 4]
    geom = po.PAGES32
    for k, shift, ok in ((0, 5, False), (1, 4, False), (2, 3, True)):
        mask = (1 << k) - 1
        offs = po.lane_offsets(ext, ds, 32, 4, 0, shift, mask)
        banks = [(4 * tx + (0 ^ ((tx >> shift) & mask))) % 32 for tx in range(32)]
        assert [o % 32 for o in offs] == banks
        assert po.step_conflict_free(offs, 4, geom) == ok
        if k == 0:
            assert all(banks.count(b) == 4 for b in set(banks))
        if k == 2:
            assert sorted(banks) == list(range(32))


def test_whole_tensor_shard():
    g = goldens.sf_ir()
    e, s, d = po.shard((2, 1, 4, 32), (128, 128, 32, 1), (128, 128, 1, 4))
    assert (e, s, d) == ([2, 4, 32], [128, 32, 1], [128, 1, 4])
    assert po.canonicalize((2, 1, 4, 32), (128, 128, 32, 1)) == ([256], [1])
    assert po.canonicalize((2, 1, 4, 32), (128, 128, 1, 4)) == ([2, 4, 32], [128, 1, 4])
    # row-major vs column-major 128x64 tile: nothing merges (no common chain)
    assert po.shard((128, 64), (64, 1), (1, 128)) == ([128, 64], [64, 1], [1, 128])
    assert po.canonicalize((128, 64), (64, 1)) == ([8192], [1])


@pytest.mark.parametrize("w,ext,ss,ds,reason", [
    (3, (4, 32), (32, 1), (1, 4), po.REASON_WIDTH),
    (32, (4, 32), (32, 1), (1, 4), po.REASON_WIDTH),
    (4, (4, 32), (32, -1), (1, 4), po.REASON_LAYOUT),
    (4, (4, 32), (32, 1), (0, 4), po.REASON_LAYOUT),
    (4, (4, 32), (32, 1), (1, 2), po.REASON_LAYOUT),
    (4, (3, 7), (7, 1), (1, 3), po.REASON_LAYOUT),
])
def test_declines(w, ext, ss, ds, reason):
    assert po.plan(w, ext, ss, ds).reason == reason


def test_result_independent_of_k():
    """Executing the per-lane program with any valid (shift, mask) gives the oracle's result."""
    rng = np.random.default_rng(5)
    cases = [((4, 32), (32, 1), (1, 4)), ((8, 32), (32, 1), (1, 8)), ((2, 4, 16), (64, 16, 1), (64, 1, 4)),
             ((16, 8), (1, 16), (8, 1))]
    for ext, ss, ds in cases:
        n = int(np.prod(ext))
        P = n // 32
        src = [int(v) for v in synth.random_bytes(0x99, n * 4).view(np.uint32)]
        ref = np.zeros(n, dtype=np.uint32)
        oracle.permute(np.array(src, dtype=np.uint32).view(np.uint8), ref.view(np.uint8), 4, ext, ss, ds)
        e, s, d = po.shard(ext, ss, ds)
        for k in po.k_candidates(P, 32):
            out = po.simulate_warp_program(src, [None] * n, e, s, d, P, 5 - k, (1 << k) - 1)
            assert out == [int(v) for v in ref]
        # in place: the same list as source and destination
        buf = list(src)
        po.simulate_warp_program(buf, buf, e, s, d, P, 3, 3 if P >= 4 else P - 1)
        assert buf == [int(v) for v in ref]


# planted mistakes in the plan oracle: each must break some pin


def _mutants():
    def only_read_phase(extent, src_str, dst_str, w, P, geom=po.PAGES32, src_swz=None, dst_swz=None):
        lanes = geom.lanes
        for k in po.k_candidates(P, lanes):
            mask, shift = (1 << k) - 1, po._log2(lanes) - k
            if po.phase_conflict_free(extent, src_str, w, lanes, P, shift, mask, geom):
                return k, shift, mask
        return None

    def shift_off_by_one(extent, src_str, dst_str, w, P, geom=po.PAGES32, src_swz=None, dst_swz=None):
        lanes = geom.lanes
        for k in po.k_candidates(P, lanes):
            mask, shift = (1 << k) - 1, max(0, po._log2(lanes) - k - 1)
            if (po.phase_conflict_free(extent, src_str, w, lanes, P, shift, mask, geom)
                    and po.phase_conflict_free(extent, dst_str, w, lanes, P, shift, mask, geom)):
                return k, shift, mask
        return None

    def column_major_decompose(n, extent):
        digits = [0] * len(extent)
        for i in range(len(extent)):
            digits[i] = n % extent[i]
            n //= extent[i]
        return digits

    def word_granular_banks(offsets, w, geom):
        seen = {}
        for o in offsets:
            word = o * w // 4
            if seen.get(word % 32, word) != word:
                return False
            seen[word % 32] = word
        return True

    return {
        "only_read_phase": ("choose_xor_k", only_read_phase),
        "shift_off_by_one": ("choose_xor_k", shift_off_by_one),
        "column_major_decompose": ("decompose", column_major_decompose),
        "same_word_not_a_conflict": ("step_conflict_free", word_granular_banks),
    }


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_plan_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(po, attr, fn)
    assert not all(pin() for pin in PINS), name


# --------------------------------------------------------------------------
# swizzled operands (the bank model sees swizzled offsets)


def test_swizzle_offset_division_form():
    from tests.test_oracle_swizzle_pins import swz_divmod
    rng = np.random.default_rng(17)
    for _ in range(500):
        bits = int(rng.integers(1, 5))
        base = int(rng.integers(0, 5))
        shift = int(rng.integers(bits, 7))
        m = int(rng.integers(0, 1 << 30))
        assert po.swizzle_offset((bits, base, shift), m) == swz_divmod(bits, base, shift, m)
    assert po.swizzle_offset(None, 77) == 77


def test_swizzled_destination_makes_the_transpose_conflict_free_unrotated():
    """32 x 32 fp32 transpose as one region.  Plain, lane l's write at step j
    goes to offset j + 32 l, bank j for every lane: only a full XOR (k = 5)
    spreads it.  With the destination swizzled by (5, 0, 5) the offset is
    (j ^ l) + 32 l, bank j ^ l, distinct across lanes: k = 0 suffices, and the
    reads (offset 32 j + l, bank l) stay conflict-free."""
    p = po.plan(4, (32, 32), (32, 1), (1, 32))
    assert p.ok and (p.k, p.shift, p.mask) == (5, 0, 31)
    q = po.plan(4, (32, 32), (32, 1), (1, 32), dst_swz=(5, 0, 5))
    assert q.ok and q.k == 0
    # Swizzling the source instead: the read bank becomes l ^ j, so every XOR
    # that spreads the writes (j depends on the lane) folds the reads together,
    # and k = 0 leaves the writes on one bank: no k.
    r = po.plan(4, (32, 32), (32, 1), (1, 32), src_swz=(5, 0, 5))
    assert not r.ok and r.reason == po.REASON_NO_K
