"""The workloads the tests and the benchmark run, as plain shape/stride data.

Each entry is a call in the library's form: element width in bytes, extents,
source strides, destination strides (all in elements), element offsets
(src, dst) and a contiguous batch count.  Seeds are 0x5EED0000 + 16 * case
number + sub-case.  Nothing here computes an address.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    w: int
    extents: Tuple[int, ...]
    src_strides: Tuple[int, ...]
    dst_strides: Tuple[int, ...]
    offsets: Tuple[int, int] = (0, 0)
    batch: int = 1
    seed: int = 0
    specials: bool = False   # force fp32 special encodings into the input
    inplace: bool = False    # source and destination are one buffer
    src_swizzle: Optional[Tuple[int, int, int]] = None   # (bits, base, shift) or None
    dst_swizzle: Optional[Tuple[int, int, int]] = None

    @property
    def elements(self) -> int:
        n = self.batch
        for e in self.extents:
            n *= e
        return n

    @property
    def bytes_moved(self) -> int:
        """Algorithmic bytes: every element read once and written once."""
        return 2 * self.elements * self.w


def _seed(case: int, sub: int = 0) -> int:
    return 0x5EED0000 + 16 * case + sub


# permute_layout page, "Demonstration program": two pipeline stages of a
# (1, 4, 32) fp32 scale-factor block, (128,128,32,1) -> (128,128,1,4).
SF_WORKED = Workload("sf_worked_example_2x1x4x32_f32", 4, (2, 1, 4, 32),
                     (128, 128, 32, 1), (128, 128, 1, 4), seed=_seed(1))

# 2**20 independent 4x32 fp32 tiles, contiguous batch (tile stride 128).
SF_BATCHED = Workload("sf_transpose_2^20x4x32_f32", 4, (4, 32), (32, 1), (1, 4),
                      batch=1 << 20, seed=_seed(2), specials=True)

# One GPU's share of the batched transpose when the batch is split over 8
# GPUs: 2^17 tiles, 64 MiB each way (small enough for the Infinity Cache, so
# the benchmark's buffer rotation keeps every launch cold).
SF_SHARE_OF_8 = Workload("sf_transpose_2^17x4x32_f32", 4, (4, 32), (32, 1), (1, 4),
                         batch=1 << 17, seed=_seed(2, 4), specials=True)

# 65536 tiles of 128x64 fp16: row-major (64,1) -> column-major (1,128).
TILE_128x64 = Workload("tile_65536x128x64_f16_rowmajor_to_colmajor", 2, (128, 64), (64, 1),
                       (1, 128), batch=65536, seed=_seed(3))


def mixed_width(w: int) -> Workload:
    """(64,128,32,32) permuted by axis order (0,2,3,1); destination is the
    row-major layout of the permuted shape (64,32,32,128)."""
    sub = {1: 0, 2: 1, 4: 2, 8: 3}[w]
    return Workload(f"axes0231_64x128x32x32_w{w}", w, (64, 128, 32, 32),
                    (131072, 1024, 32, 1), (131072, 1, 4096, 128), seed=_seed(4, sub))


BF16_16K = Workload("transpose_16384x16384_bf16", 2, (16384, 16384), (16384, 1), (1, 16384),
                    seed=_seed(5, 0))
W16_4K = Workload("transpose_4096x4096_16B", 16, (4096, 4096), (4096, 1), (1, 4096),
                  seed=_seed(5, 1))

# Outer-axis permutation with contiguous inner runs: (64,128,32,32) by axis
# order (1,0,2,3); both sides keep the last two axes as one 4 KiB run.
OUTER_PERM = Workload("axes1023_64x128x32x32_f32_runs", 4, (64, 128, 32, 32),
                      (131072, 1024, 32, 1), (1024, 65536, 32, 1), seed=_seed(6))

# The same re-layout for 1-byte (e8m0 / fp8) and 2-byte (fp16) scale factors.
SF_U8 = Workload("sf_transpose_2^20x4x32_u8", 1, (4, 32), (32, 1), (1, 4), batch=1 << 20, seed=_seed(2, 2))
SF_F16 = Workload("sf_transpose_2^20x4x32_f16", 2, (4, 32), (32, 1), (1, 4), batch=1 << 20, seed=_seed(2, 3))
# An array of 2^24 float4 records to one array per component (AoS -> SoA).
AOS_TO_SOA = Workload("aos_to_soa_2^24x4_f32", 4, (1 << 24, 4), (4, 1), (1, 1 << 24), seed=_seed(7))
# An array of 2^24 float3 (xyz) records to 3 field arrays.
AOS3_TO_SOA = Workload("aos_to_soa_2^24x3_f32", 4, (1 << 24, 3), (3, 1), (1, 1 << 24), seed=_seed(7, 1))
# The 16384^2 bf16 transpose with source rows one element longer than the
# row: no row but the first starts on a 16-byte boundary.
BF16_16K_ODD_PITCH = Workload("transpose_16384x16384_bf16_src_pitch_16385", 2, (16384, 16384), (16385, 1),
                              (1, 16384), seed=_seed(7, 2))
# The SF transpose into XOR-swizzled destination tiles: the 16-byte chunk
# index of each 128-element tile (bits 2..3 of the offset) is XORed with bits
# 5..6; the swizzle period is one tile.
SF_SWIZZLED = Workload("sf_transpose_2^20x4x32_f32_to_swizzled", 4, (4, 32), (32, 1), (1, 4),
                       batch=1 << 20, seed=_seed(2, 1), specials=True, dst_swizzle=(2, 2, 3))
# The fp16 tiles into MMA-style swizzled column-major tiles: 16-byte chunks of
# each 256-byte destination row XORed with the row index (bits 3..5 ^= 7..9).
TILE_SWIZZLED = Workload("tile_65536x128x64_f16_to_swizzled_colmajor", 2, (128, 64), (64, 1), (1, 128),
                         batch=65536, seed=_seed(3, 1), dst_swizzle=(3, 3, 4))
# The 16384^2 bf16 transpose with source and destination in one buffer.
BF16_16K_INPLACE = Workload("transpose_16384x16384_bf16_inplace", 2, (16384, 16384), (16384, 1), (1, 16384),
                            seed=_seed(5, 2), inplace=True)
# Not workloads of the method: identity layouts (plain copies) of known size,
# used to calibrate the HBM byte counters (512 MiB) and as same-size copy
# references for the counter profiles of the small permutes.
COPY_CALIBRATION = Workload("identity_copy_512MiB_u32", 4, (1 << 27,), (1,), (1,), seed=0x5EED0100)
COPY_REFERENCES = [Workload(f"identity_copy_{m}MiB_u32", 4, (m << 18,), (1,), (1,), seed=0x5EED0100 + m)
                   for m in (8, 16, 32, 64)] + [COPY_CALIBRATION]

ALL = ([SF_WORKED, SF_BATCHED, SF_SHARE_OF_8, TILE_128x64] + [mixed_width(w) for w in (1, 2, 4, 8)]
       + [BF16_16K, W16_4K, OUTER_PERM, SF_SWIZZLED, TILE_SWIZZLED, SF_U8, SF_F16, AOS_TO_SOA, AOS3_TO_SOA,
          BF16_16K_ODD_PITCH])
INPLACE = [BF16_16K_INPLACE]


def scaled(wl: Workload, batch: int = None, extents=None) -> Workload:
    """The same layouts on a smaller batch or extents (for CPU-sized parity cases)."""
    from dataclasses import replace
    kw = {}
    if batch is not None:
        kw["batch"] = batch
    if extents is not None:
        kw["extents"] = tuple(extents)
    return replace(wl, **kw)
