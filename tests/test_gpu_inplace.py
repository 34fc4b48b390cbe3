"""GPU parity of in-place square transposes (src and dst the same memory).

Mirrored tiles are swapped pairwise, each pair by one workgroup that reads
both tiles before writing either.  The expected buffer is the input with the
oracle's permutation written over it: elements outside the layout (row
padding, gaps between batch items) must keep their input bytes.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def square(n, pitch, batch=1, gap=0):
    """(extents, src strides, dst strides, elements) of `batch` n x n transposes
    with rows `pitch` elements apart and `gap` spare elements after each item."""
    item = n * pitch + gap
    ext = (batch, n, n) if batch > 1 else (n, n)
    ss = ((item, pitch, 1) if batch > 1 else (pitch, 1))
    ds = ((item, 1, pitch) if batch > 1 else (1, pitch))
    return ext, ss, ds, batch * item


def run_inplace(name, w, n, pitch, batch=1, gap=0, offset=0, seed=3, expect_kernel="swap"):
    torch = _torch()
    ext, ss, ds, elems = square(n, pitch, batch, gap)
    print(f"\n[case] in place {name}: w={w} ext={ext} ss={ss} ds={ds} offset={offset}", flush=True)
    nbytes = (offset + elems) * w
    x = synth.random_bytes(seed, nbytes).copy()
    ref = x.copy()
    oracle.permute(x, ref, w, ext, ss, ds, (offset, offset), 1)
    if expect_kernel is not None:
        p = tpl.tpl_plan(w, ext, ss, ds, (offset, offset), 1, geometry=tpl.TPL_GEOM_GFX950_INPLACE)
        assert p.kernel == expect_kernel, p
    buf = torch.from_numpy(x).cuda()
    tpl.permute(buf, buf, ext, ss, ds, offset, offset, 1, dtype_bytes=w)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    if not np.array_equal(got, ref):
        diff = np.flatnonzero(got != ref)
        raise AssertionError(f"{name}: {diff.size} bytes differ; first at byte {diff[0]}")


CASES = [
    # name, w, n, pitch, batch, gap, offset (elements)
    ("u8_512", 1, 512, 512, 1, 0, 0),
    ("u8_300_ragged", 1, 300, 300, 1, 0, 0),
    ("u16_1024", 2, 1024, 1024, 1, 0, 0),
    ("u16_200_pitch256", 2, 200, 256, 1, 0, 0),
    ("u32_1000_ragged", 4, 1000, 1000, 1, 0, 0),
    ("u32_64_one_tile", 4, 64, 64, 1, 0, 0),
    ("u32_8_below_tile", 4, 8, 8, 5, 0, 0),
    ("u32_100_pitch101_unaligned", 4, 100, 101, 1, 0, 0),
    ("u32_96_offset_3", 4, 96, 96, 1, 0, 3),
    ("u64_96_batched", 8, 96, 96, 3, 16, 0),
    ("u64_256", 8, 256, 256, 1, 0, 0),
    ("16B_100_ragged", 16, 100, 100, 1, 0, 0),
    ("16B_512", 16, 512, 512, 1, 0, 0),
    ("u16_65_batched_gap", 2, 65, 72, 4, 9, 0),
    # tile counts past one 8 x 8-tile block: 10 (2 blocks, the second partly
    # outside), 21 (3 blocks, ragged tiles), 40 (5 blocks, batched)
    ("u8_1200_two_blocks", 1, 1200, 1200, 1, 0, 0),
    ("16B_330_three_blocks_ragged", 16, 330, 330, 1, 0, 0),
    ("u16_2560_five_blocks_batched", 2, 2560, 2560, 2, 64, 0),
    # items of one element tile with unaligned rows: the element-tile kernel
    # reads an item's 16-byte chunks (some shared with the neighbouring
    # items) before it writes any of the item
    ("u8_100_pitch101_batched_one_tile", 1, 100, 101, 7, 0, 0),
    ("u16_60_pitch61_batched_one_tile", 2, 60, 61, 9, 3, 1),
    # the same with enough items for the tall element tiles
    ("u8_100_pitch101_4096_items_tall", 1, 100, 101, 4096, 0, 0),
    ("u16_60_pitch61_4096_items_tall", 2, 60, 61, 4096, 3, 1),
]

ONE_TILE = {"u32_64_one_tile": "lds", "u8_100_pitch101_batched_one_tile": "etile",
            "u16_60_pitch61_batched_one_tile": "etile", "u8_100_pitch101_4096_items_tall": "etile",
            "u16_60_pitch61_4096_items_tall": "etile"}


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_inplace_square_transpose(case):
    name, w, n, pitch, batch, gap, offset = case
    # items of one tile: the ordinary tile kernels already read before they write
    kernel = ONE_TILE.get(name, "swap")
    run_inplace(name, w, n, pitch, batch, gap, offset, expect_kernel=kernel)


def test_inplace_bf16_16384_full_size():
    run_inplace("bf16_16384x16384", 2, 16384, 16384)


def test_inplace_twice_is_identity():
    """A square transpose applied twice in place restores the buffer."""
    torch = _torch()
    print("\n[case] in place twice: u32 4096 x 4096", flush=True)
    n = 4096
    x = synth.random_bytes(11, n * n * 4).copy()
    buf = torch.from_numpy(x).cuda()
    for _ in range(2):
        tpl.permute(buf, buf, (n, n), (n, 1), (1, n), dtype_bytes=4)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), x)


def test_inplace_non_square_is_refused_and_untouched():
    torch = _torch()
    print("\n[case] in place non-square -> TPL_E_ALIAS", flush=True)
    x = synth.random_bytes(12, 200 * 100 * 4).copy()
    buf = torch.from_numpy(x).cuda()
    with pytest.raises(tpl.TplError) as e:
        tpl.permute(buf, buf, (100, 200), (200, 1), (1, 100), dtype_bytes=4)
    assert e.value.status == tpl.TPL_E_ALIAS
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), x)
