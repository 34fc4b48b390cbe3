"""Plan oracle for permute_layout: canonicalise, regroup, P, and the XOR-k search.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library's planner; it restates the method's host-side steps in plain Python so
the library's planner can be checked against it.

The steps follow the permute_layout page, section "Algorithm":

1. Align the two layouts: slice to the region, canonicalise each side, and when
   the shard structures differ regroup the source to the destination's shape;
   the iteration extent and both stride lists come from the resulting shard.
   P = prod(extent) / lanes.
2. Choose the XOR swizzle: simulate the shared-memory bank pattern of both
   phases for k = 0, 1, ... and take the smallest k that makes both phases
   conflict-free; otherwise decline.
3. The per-lane program: at unrolled step r a lane visits iteration
   j = r ^ ((lane >> shift) & mask), decomposes lane + j * lanes over the
   extent (row-major, last axis fastest), and projects the digits onto the
   side's strides.

Readings where the pages are silent (each listed in the design notes):

* canonical form: modes of extent 1 are dropped and neighbours i, i+1 merge
  when stride_i == extent_{i+1} * stride_{i+1}; modes are never reordered;
* regrouping: the shard merges neighbours only where *both* sides merge (the
  coarsest common refinement); with a linear source and a transposed
  destination this is exactly "the source regrouped to the destination";
* k ranges over 0 .. min(floor(log2 P), log2 lanes) with 2**k dividing P, so
  the XOR keeps j inside [0, P); mask = 2**k - 1 and shift = log2(lanes) - k
  (the key is the top k bits of the lane id);
* P not an integer: decline;
* the conflict model of the pages' hardware: 32 banks of 4 bytes, one step r
  of the whole warp is one access; bank = floor(byte_offset / 4) mod 32 and
  two lanes in one bank conflict even inside one 4-byte word (that is what
  lets stride-1 sub-4-byte reads fail, as the "How inputs change the
  algorithm" table says).  An element of w > 4 bytes covers w/4 consecutive
  banks and the warp is served in groups of 128/w lanes.

Parity unpinned: that last sentence (elements of 8 and 16 bytes).  No value on
the pages fixes it, and the tests' brute-force simulator restates the same
reading, so for those widths this oracle is checked against itself only.  The
1- to 4-byte model is pinned by the pages' worked example and declines.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

# Decline reasons, in the order of the pages' predicate list ("What it accepts").
REASON_WIDTH = "unsupported dtype byte width"
REASON_LAYOUT = "layouts must slice/canonicalize"
REASON_NO_K = "no XOR k makes both phases bank-conflict-free"
REASON_EXTENT = "extent mismatch"
REASON_DTYPE = "dtype mismatch"


@dataclass
class Geometry:
    """Bank model used by the k search: the pages' shared memory.

    One unrolled step of the whole warp is split into passes of
    ``pass_lanes(w)`` consecutive lanes; inside one pass no two lanes may use
    the same bank, even when they touch the same word.
    """

    lanes: int = 32          # lanes that run one unrolled step together
    banks: int = 32          # number of banks
    bank_bytes: int = 4      # bytes per bank

    def pass_lanes(self, w: int) -> int:
        words = max(1, w // self.bank_bytes)
        return max(1, min(self.lanes, self.banks // words))


PAGES32 = Geometry()


@dataclass
class Plan:
    ok: bool
    reason: str = ""
    extent: List[int] = field(default_factory=list)
    src_str: List[int] = field(default_factory=list)
    dst_str: List[int] = field(default_factory=list)
    P: int = 0
    k: int = -1
    shift: int = 0
    mask: int = 0


def _log2(x: int) -> int:
    return x.bit_length() - 1


def drop_unit_modes(extents, src, dst):
    """Drop modes of extent 1 (they contribute nothing to any address)."""
    keep = [i for i, e in enumerate(extents) if e != 1]
    return [extents[i] for i in keep], [src[i] for i in keep], [dst[i] for i in keep]


def mergeable(extents: Sequence[int], strides: Sequence[int], i: int) -> bool:
    """Neighbours i, i+1 form one longer run when stride_i = extent_{i+1} * stride_{i+1}."""
    return strides[i] == extents[i + 1] * strides[i + 1]


def canonicalize(extents: Sequence[int], strides: Sequence[int]) -> Tuple[List[int], List[int]]:
    """Canonical form of one side: unit modes dropped, mergeable neighbours merged."""
    e = [x for x in extents if x != 1]
    s = [strides[i] for i, x in enumerate(extents) if x != 1]
    if not e:
        return [1], [1]
    out_e, out_s = [e[0]], [s[0]]
    for i in range(1, len(e)):
        if out_s[-1] == e[i] * s[i]:
            out_e[-1] *= e[i]
            out_s[-1] = s[i]
        else:
            out_e.append(e[i])
            out_s.append(s[i])
    return out_e, out_s


def shard(extents, src, dst):
    """Step 1: the common shard (merge only where both sides merge)."""
    e, s, d = drop_unit_modes(list(extents), list(src), list(dst))
    if not e:
        return [1], [1], [1]
    oe, os_, od = [e[0]], [s[0]], [d[0]]
    for i in range(1, len(e)):
        if os_[-1] == e[i] * s[i] and od[-1] == e[i] * d[i]:
            oe[-1] *= e[i]
            os_[-1] = s[i]
            od[-1] = d[i]
        else:
            oe.append(e[i])
            os_.append(s[i])
            od.append(d[i])
    return oe, os_, od


def decompose(n: int, extent: Sequence[int]) -> List[int]:
    """Row-major mixed-radix digits of n over extent (last axis fastest)."""
    digits = [0] * len(extent)
    for i in range(len(extent) - 1, -1, -1):
        digits[i] = n % extent[i]
        n //= extent[i]
    return digits


def project(idx: Sequence[int], strides: Sequence[int]) -> int:
    return sum(i * s for i, s in zip(idx, strides))


def swizzle_offset(z, m: int) -> int:
    """An operand's XOR swizzle (bits, base, shift) of a layout offset: the
    bits-wide field at bit base + shift is XORed into the field at bit base.
    None or bits == 0: the plain layout.  (The pages allocate such tiles for
    MMA operands but leave the function to the allocator; this is the usual
    form.)"""
    if z is None or z[0] == 0:
        return m
    bits, base, shift = z
    return m ^ (((m >> (base + shift)) & ((1 << bits) - 1)) << base)


def lane_offsets(extent, strides, lanes, P, r, shift, mask, swz=None) -> List[int]:
    """Element offset each lane touches at unrolled step r (the per-lane program)."""
    out = []
    for lane in range(lanes):
        j = r ^ ((lane >> shift) & mask)
        out.append(swizzle_offset(swz, project(decompose(lane + j * lanes, extent), strides)))
    return out


def step_conflict_free(offsets: Sequence[int], w: int, geom: Geometry) -> bool:
    """One step of one phase: does any bank serve two lanes within one pass?"""
    words = max(1, w // geom.bank_bytes)
    lanes_per_pass = geom.pass_lanes(w)
    for p0 in range(0, len(offsets), lanes_per_pass):
        seen = set()
        for o in offsets[p0:p0 + lanes_per_pass]:
            word0 = (o * w) // geom.bank_bytes
            for k in range(words):
                bank = (word0 + k) % geom.banks
                if bank in seen:
                    return False
                seen.add(bank)
    return True


def phase_conflict_free(extent, strides, w, lanes, P, shift, mask, geom, swz=None) -> bool:
    return all(
        step_conflict_free(lane_offsets(extent, strides, lanes, P, r, shift, mask, swz), w, geom)
        for r in range(P)
    )


def k_candidates(P: int, lanes: int):
    """k in 0 .. min(floor(log2 P), log2 lanes) with 2**k dividing P."""
    kmax = min(_log2(P), _log2(lanes))
    for k in range(kmax + 1):
        if P % (1 << k) == 0:
            yield k


def choose_xor_k(extent, src_str, dst_str, w, P, geom: Geometry = PAGES32, src_swz=None, dst_swz=None):
    """Step 2: smallest k whose (shift, mask) makes both phases conflict-free."""
    lanes = geom.lanes
    for k in k_candidates(P, lanes):
        mask = (1 << k) - 1
        shift = _log2(lanes) - k
        if (phase_conflict_free(extent, src_str, w, lanes, P, shift, mask, geom, src_swz)
                and phase_conflict_free(extent, dst_str, w, lanes, P, shift, mask, geom, dst_swz)):
            return k, shift, mask
    return None


def dst_injective(extents, dst) -> bool:
    """Sufficient test: sorted by stride, each mode's stride exceeds the span below it."""
    modes = sorted((s, e) for e, s in zip(extents, dst) if e != 1)
    span = 0
    for s, e in modes:
        if s <= span:
            return False
        span += (e - 1) * s
    return True


def plan(w: int, extents, src_strides, dst_strides, geom: Geometry = PAGES32, src_swz=None,
         dst_swz=None) -> Plan:
    """The whole host-side method for one warp region, in the pages' order.
    Swizzled operands (outside the pages' method): the bank model sees the
    swizzled offsets."""
    if w not in (1, 2, 4, 8, 16):
        return Plan(False, REASON_WIDTH)
    if any(e < 1 for e in extents):
        return Plan(False, REASON_LAYOUT)
    if any(s < 0 for s in list(src_strides) + list(dst_strides)):
        return Plan(False, REASON_LAYOUT)
    if not dst_injective(extents, dst_strides):
        return Plan(False, REASON_LAYOUT)
    ext, ss, ds = shard(extents, src_strides, dst_strides)
    total = 1
    for e in ext:
        total *= e
    if total % geom.lanes:
        return Plan(False, REASON_LAYOUT, ext, ss, ds)
    P = total // geom.lanes
    got = choose_xor_k(ext, ss, ds, w, P, geom, src_swz, dst_swz)
    if got is None:
        return Plan(False, REASON_NO_K, ext, ss, ds, P)
    k, shift, mask = got
    return Plan(True, "", ext, ss, ds, P, k, shift, mask)


def simulate_warp_program(src: List[int], dst: List[int], extent, src_str, dst_str,
                          P, shift, mask, lanes=32, src_off=0, dst_off=0):
    """Execute the two register-staged phases on Python lists, lane by lane.

    Phase 1 fills every lane's registers through the source layout; only then
    does phase 2 write them through the destination layout (the warp-sync in
    between), so src and dst may be the same list.
    """
    regs = [[None] * P for _ in range(lanes)]
    for lane in range(lanes):
        for r in range(P):
            j = r ^ ((lane >> shift) & mask)
            regs[lane][r] = src[src_off + project(decompose(lane + j * lanes, extent), src_str)]
    for lane in range(lanes):
        for r in range(P):
            j = r ^ ((lane >> shift) & mask)
            dst[dst_off + project(decompose(lane + j * lanes, extent), dst_str)] = regs[lane][r]
    return dst
