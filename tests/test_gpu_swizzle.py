"""GPU parity with XOR-swizzled operands, against the oracle, byte for byte.

Every kernel family that accepts a swizzled side is run: the quad kernel
(SF tiles), the LDS tile kernel (full and ragged tiles, every width), the
run copy, the element-wise kernel (granules narrower than 16 bytes), and the
staged half-wave program.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl
from tests.test_gpu_parity import run_case

pytestmark = pytest.mark.gpu


CASES = [
    # name, w, ext, ss, ds, batch, src swizzle, dst swizzle, kernel
    ("sf_dst_16B_granules", 4, (4, 32), (32, 1), (1, 4), 4097, None, (3, 2, 3), "quad"),
    ("sf_src_swizzled", 4, (4, 32), (32, 1), (1, 4), 1023, (2, 2, 3), None, "quad"),
    ("sf_narrow_quads_both", 4, (4, 8), (8, 1), (1, 4), 999, (1, 2, 2), (1, 2, 3), "quad"),
    ("sf_8B_granules_elementwise", 4, (4, 32), (32, 1), (1, 4), 513, None, (3, 1, 3), "gather"),
    ("sf_u8_dst_swizzled", 1, (4, 32), (32, 1), (1, 4), 1025, None, (2, 4, 3), "quad"),
    ("sf_u16_src_swizzled", 2, (4, 32), (32, 1), (1, 4), 1027, (2, 3, 3), None, "quad"),
    ("aos_to_soa_f16x8_split_dst_swizzled", 2, (4096, 8), (8, 1), (1, 4096), 3, None, (2, 3, 4), "quad"),
    ("f16_tiles_mma_colmajor", 2, (128, 64), (64, 1), (1, 128), 17, None, (3, 3, 4), "lds"),
    ("u8_256_both", 1, (256, 256), (256, 1), (1, 256), 2, (3, 4, 4), (3, 4, 5), "lds"),
    ("u64_src", 8, (64, 64), (64, 1), (1, 64), 3, (2, 1, 3), None, "lds"),
    ("16B_both", 16, (64, 64), (64, 1), (1, 64), 2, (3, 0, 3), (3, 0, 6), "lds"),
    ("16B_8x8_ragged", 16, (8, 8), (8, 1), (1, 8), 5, None, (3, 0, 3), "lds"),
    ("bf16_ragged_tiles", 2, (96, 72), (72, 1), (1, 96), 3, (2, 3, 3), (3, 3, 3), "lds"),
    ("u32_runs_copy", 4, (64, 64), (64, 1), (64, 1), 8, None, (2, 1, 4), "copy"),
    ("u32_runs_16B", 4, (16, 8, 64), (64, 1024, 1), (512, 64, 1), 2, (2, 2, 6), (2, 2, 4), "copy"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_swizzled_matches_oracle(case):
    name, w, ext, ss, ds, batch, zs, zd, kernel = case
    run_case(name, w, ext, ss, ds, (0, 0), batch, seed=0x5712, expect_kernel=kernel, zs=zs, zd=zd)


def test_swizzled_unaligned_offsets_go_elementwise():
    run_case("sf_dst_swizzled_offset_3", 4, (4, 32), (32, 1), (1, 4), (0, 3), 129, seed=5,
             expect_kernel="gather", zd=(3, 2, 3))


def test_swizzled_round_trip():
    """Into a swizzled tile and back out with the inverse layouts: the input again."""
    torch = _torch()
    print("\n[case] swizzled round trip, fp16 128x64 tiles x 256", flush=True)
    n = 256 * 128 * 64
    x = synth.random_bytes(21, n * 2).copy()
    a = torch.from_numpy(x).cuda()
    b = torch.empty_like(a)
    c = torch.empty_like(a)
    tpl.permute(b, a, (128, 64), (64, 1), (1, 128), batch=256, dtype_bytes=2, dst_swizzle=(3, 3, 4))
    tpl.permute(c, b, (128, 64), (1, 128), (64, 1), batch=256, dtype_bytes=2, src_swizzle=(3, 3, 4))
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), x)
    assert not np.array_equal(b.cpu().numpy()[: 64 * 128 * 2], x[: 64 * 128 * 2])


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def run_staged_swizzled(name, w, ext, ss, ds, batch, zs, zd, xor_k=-1):
    torch = _torch()
    print(f"\n[case] staged swizzled {name}: w={w} ext={ext} zs={zs} zd={zd} batch={batch} k={xor_k}", flush=True)
    span_s = 1 + sum((e - 1) * s for e, s in zip(ext, ss))
    span_d = 1 + sum((e - 1) * s for e, s in zip(ext, ds))
    x = synth.random_bytes(31, batch * span_s * w).copy()
    ref = np.full(batch * span_d * w, 0xA5, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, (0, 0), batch, zs, zd)
    s = torch.from_numpy(x).cuda()
    d = torch.full((ref.size,), 0xA5, dtype=torch.uint8, device="cuda")
    st = tpl.tpl_permute_staged(s.data_ptr(), d.data_ptr(), w, ext, ss, ds, (0, 0), batch, xor_k,
                                torch.cuda.current_stream().cuda_stream, zs, zd)
    assert st == tpl.TPL_OK, tpl.tpl_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), ref), name


def test_staged_swizzled_destination_transpose():
    """32 x 32 fp32 transposes into (5, 0, 5)-swizzled tiles: the planner's k
    is 0 (the swizzle already spreads the banks), and any forced k gives the
    same bytes."""
    p = tpl.tpl_plan(4, (32, 32), (32, 1), (1, 32), geometry=tpl.TPL_GEOM_GFX950_HALFWAVE, dst_swizzle=(5, 0, 5))
    assert p.ok and p.k == 0
    run_staged_swizzled("f32_32x32_dst", 4, (32, 32), (32, 1), (1, 32), 65, None, (5, 0, 5))
    run_staged_swizzled("f32_32x32_dst_k5", 4, (32, 32), (32, 1), (1, 32), 65, None, (5, 0, 5), xor_k=5)


def test_staged_swizzled_fp16_tiles():
    run_staged_swizzled("f16_16x64_both", 2, (16, 64), (64, 1), (1, 16), 33, (3, 3, 3), (2, 3, 4))
