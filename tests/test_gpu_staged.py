"""GPU parity of tpl_permute_staged: the pages' warp program, one batch item per
32-lane half-wave, staged through LDS (tpl_wave.h), against the CPU oracle.

The result must not depend on the XOR swizzle (it only reorders accesses), so
every case also runs with the swizzle forced off (k = 0).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def cosize(extents, strides):
    return 1 + sum((e - 1) * s for e, s in zip(extents, strides))


def run_staged(name, w, ext, ss, ds, batch, xor_k=-1, seed=1):
    torch = _torch()
    print(f"\n[case] staged {name}: w={w} ext={ext} ss={ss} ds={ds} batch={batch} xor_k={xor_k}", flush=True)
    ns, nd = batch * cosize(ext, ss) * w, batch * cosize(ext, ds) * w
    x = synth.random_bytes(seed, ns).copy()
    ref = np.full(nd, SENTINEL, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, (0, 0), batch)
    s = torch.from_numpy(x).cuda()
    d = torch.full((nd,), SENTINEL, dtype=torch.uint8, device="cuda")
    st = tpl.tpl_permute_staged(s.data_ptr(), d.data_ptr(), w, ext, ss, ds, (0, 0), batch, xor_k,
                                torch.cuda.current_stream().cuda_stream)
    assert st == tpl.TPL_OK, tpl.tpl_last_error()
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    assert np.array_equal(got, ref), f"{name}: {int(np.count_nonzero(got != ref))} bytes differ"


CASES = [
    ("worked_example_regions", 4, (1, 4, 32), (128, 32, 1), (128, 1, 4), 2),
    ("sf_fp32", 4, (4, 32), (32, 1), (1, 4), 4097),
    ("sf_fp16", 2, (4, 32), (32, 1), (1, 4), 1001),
    ("sf_u8", 1, (4, 32), (32, 1), (1, 4), 513),
    ("8x32_fp32", 4, (8, 32), (32, 1), (1, 8), 300),
    ("32x32_fp32", 4, (32, 32), (32, 1), (1, 32), 65),
    ("16x64_fp16", 2, (16, 64), (64, 1), (1, 16), 77),
    ("4d_axes0231_u16", 2, (2, 4, 4, 8), (128, 32, 8, 1), (128, 1, 32, 4), 33),
    # items of one 16-byte chunk per lane take the pipelined loop: several
    # full iterations per workgroup (3072 workgroups move 6144 items per
    # iteration), then a partial one with an odd item count, or none
    ("sf_fp32_pipelined_odd_tail", 4, (4, 32), (32, 1), (1, 4), 3 * 6144 + 1001),
    ("sf_fp32_pipelined_whole", 4, (4, 32), (32, 1), (1, 4), 2 * 6144),
    ("8x32_fp16_pipelined", 2, (8, 32), (32, 1), (1, 8), 6144 + 1),
    ("16x32_u8_pipelined", 1, (16, 32), (32, 1), (1, 16), 5 * 6144 - 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_staged_matches_oracle(case):
    name, w, ext, ss, ds, batch = case
    run_staged(name, w, ext, ss, ds, batch)
    run_staged(name + "_k0", w, ext, ss, ds, batch, xor_k=0)


def test_staged_plan_is_the_pages_plan_for_the_worked_example():
    p = tpl.tpl_plan(4, (1, 4, 32), (128, 32, 1), (128, 1, 4), geometry=tpl.TPL_GEOM_GFX950_HALFWAVE)
    assert (p.P, p.k, p.shift, p.mask) == (4, 2, 3, 3)


def test_staged_forced_k_runs_where_the_planner_declines():
    run_staged("sf_fp64_forced_k0", 8, (4, 32), (32, 1), (1, 4), 257, xor_k=0)
    # Source rows padded to 40 elements: the read phase's banks depend on the
    # row, so no XOR of the write phase keeps both phases conflict-free (the
    # pages' rule declines); forcing a k still computes the right result.
    p = tpl.tpl_plan(4, (4, 32), (40, 1), (1, 4), geometry=tpl.TPL_GEOM_GFX950_HALFWAVE)
    assert p.status == tpl.TPL_E_NO_K
    for k in (0, 1, 2):
        run_staged(f"padded_source_rows_forced_k{k}", 4, (4, 32), (40, 1), (1, 4), 129, xor_k=k)
