"""GPU parity: the HIP path through the C ABI against the CPU oracle, byte for byte.

Every case prints its name before touching the GPU.  Destinations start
filled with the sentinel byte 0xA5 so that a missed or stray write shows up as
a difference from the oracle, which sees the same sentinel.
"""

from __future__ import annotations

import zlib

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl, workloads

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def cosize(extents, strides):
    if any(e == 0 for e in extents):
        return 0
    return 1 + sum((e - 1) * s for e, s in zip(extents, strides))


def sizes(w, ext, ss, ds, offs, batch, zs=None, zd=None):
    ns = offs[0] + tpl._swz_reach(batch * cosize(ext, ss), zs)
    nd = offs[1] + tpl._swz_reach(batch * cosize(ext, ds), zd)
    return ns * w, nd * w


def make_input(seed, nbytes, specials=False, w=4):
    x = synth.random_bytes(seed, nbytes).copy()
    if specials and w == 4:
        synth.inject_f32_specials(x.view(np.uint32), seed ^ 0x5EC1A1)
    return x


def run_case(name, w, ext, ss, ds, offs=(0, 0), batch=1, seed=1, specials=False, expect_kernel=None,
             zs=None, zd=None):
    torch = _torch()
    print(f"\n[case] {name}: w={w} ext={tuple(ext)} ss={tuple(ss)} ds={tuple(ds)} offs={tuple(offs)} batch={batch}"
          f" swizzles={zs},{zd}", flush=True)
    nbs, nbd = sizes(w, ext, ss, ds, offs, batch, zs, zd)
    x = make_input(seed, nbs, specials, w)
    ref = np.full(nbd, SENTINEL, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, offs, batch, zs, zd)
    s = torch.from_numpy(x).cuda()
    d = torch.full((max(nbd, 1),), SENTINEL, dtype=torch.uint8, device="cuda")
    if expect_kernel is not None:
        plan = tpl.tpl_plan(w, ext, ss, ds, offs, batch, src_swizzle=zs, dst_swizzle=zd)
        assert plan.kernel == expect_kernel, plan
    tpl.permute(d, s, ext, ss, ds, offs[0], offs[1], batch, dtype_bytes=w, src_swizzle=zs, dst_swizzle=zd)
    torch.cuda.synchronize()
    got = d.cpu().numpy()[:nbd]
    if not np.array_equal(got, ref):
        diff = np.flatnonzero(got != ref)
        raise AssertionError(f"{name}: {diff.size} bytes differ; first at byte {diff[0]}")
    return got


# ---------------------------------------------------------------------------
# the workloads, on sizes the oracle finishes in well under a second


SMALL = [
    workloads.SF_WORKED,
    workloads.scaled(workloads.SF_BATCHED, batch=8192),
    workloads.scaled(workloads.TILE_128x64, batch=64),
    workloads.scaled(workloads.mixed_width(1), extents=(2, 128, 32, 32)),
    workloads.scaled(workloads.mixed_width(2), extents=(2, 128, 32, 32)),
    workloads.scaled(workloads.mixed_width(4), extents=(2, 128, 32, 32)),
    workloads.scaled(workloads.mixed_width(8), extents=(2, 128, 32, 32)),
    workloads.Workload("transpose_1024x768_bf16", 2, (1024, 768), (768, 1), (1, 1024), seed=0x5EED0050),
    workloads.Workload("transpose_256x192_16B", 16, (256, 192), (192, 1), (1, 256), seed=0x5EED0051),
    workloads.scaled(workloads.SF_SWIZZLED, batch=4097),
    workloads.scaled(workloads.SF_U8, batch=4099),
    workloads.scaled(workloads.SF_F16, batch=4101),
    workloads.scaled(workloads.TILE_SWIZZLED, batch=33),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_workload_small(wl):
    run_case(wl.name, wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
             wl.seed, wl.specials, zs=wl.src_swizzle, zd=wl.dst_swizzle)


# ---------------------------------------------------------------------------
# the workloads at full size, in the launch configuration the benchmark times


@pytest.mark.parametrize("wl", workloads.ALL, ids=lambda w: w.name)
def test_workload_full_size(wl):
    run_case(wl.name, wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
             wl.seed, wl.specials, zs=wl.src_swizzle, zd=wl.dst_swizzle)


# ---------------------------------------------------------------------------
# ragged tails, several tiles, every kernel family


RAGGED = [
    # (name, w, extents, src strides, dst strides, expected kernel); rows padded to 16 bytes
    ("lds_w1_ragged", 1, (3, 200, 333), (200 * 336, 336, 1), (333 * 208, 1, 208), "lds"),
    ("lds_w2_ragged", 2, (2, 130, 1000), (130 * 1000, 1000, 1), (1000 * 136, 1, 136), "lds"),
    ("lds_w4_ragged", 4, (3, 70, 130), (70 * 132, 132, 1), (130 * 72, 1, 72), "lds"),
    ("lds_w8_ragged", 8, (2, 33, 65), (33 * 66, 66, 1), (65 * 34, 1, 34), "lds"),
    ("lds_w2_small_tile", 2, (96, 160), (168, 1), (1, 104), "lds"),
    ("lds_w1_small_tile", 1, (80, 144), (160, 1), (1, 96), "lds"),
    ("reg16_ragged", 16, (13, 27), (27, 1), (1, 13), "reg16"),
    ("lds_w16_ragged", 16, (3, 40, 70), (40 * 70, 70, 1), (70 * 40, 1, 40), "lds"),
    ("lds_w16_big_tile_ragged", 16, (50, 200), (200, 1), (1, 50), "lds"),
    ("quad_qpr9", 4, (4, 36), (36, 1), (1, 4), "quad"),
    ("quad_padded", 4, (5, 4, 32), (160, 40, 1), (256, 1, 8), "quad"),
    ("quad_u8_narrow_batched", 1, (7, 4, 48), (256, 64, 1), (208, 1, 4), "quad"),
    ("quad_u8_wide", 1, (3, 4, 256), (1024, 256, 1), (1024, 1, 4), "quad"),
    ("quad_u16_narrow_padded_rows", 2, (9, 4, 24), (160, 40, 1), (96, 1, 4), "quad"),
    ("quad_u16_wide", 2, (5, 4, 128), (512, 128, 1), (512, 1, 4), "quad"),
    ("gather_u8_columns_apart", 1, (6, 4, 32), (128, 32, 1), (256, 1, 8), "gather"),
    ("quad_soa_to_aos_u8x16_split", 1, (16, 4096), (4096, 1), (1, 16), "quad"),
    ("quad_aos_to_soa_u16x8_split_padded", 2, (2048, 8), (8, 1), (1, 2056), "quad"),
    ("quad_aos_to_soa_f16x8", 2, (40000, 8), (8, 1), (1, 40000), "quad"),
    ("quad_aos_to_soa_u8x16_batched", 1, (2, 8192, 16), (8192 * 16, 16, 1), (8192 * 16, 1, 8192), "quad"),
    ("quad_soa_to_aos_f16x8", 2, (8, 40000), (40000, 1), (1, 8), "quad"),
    ("rec_aos_to_soa_f32x3", 4, (100003, 3), (3, 1), (1, 100004), "rec"),
    ("rec_soa_to_aos_f32x3_batched", 4, (2, 3, 50000), (150000, 50000, 1), (150000, 1, 3), "rec"),
    ("rec_rgb_to_planes", 1, (3, 65536, 3), (65536 * 3, 3, 1), (3 * 65536, 1, 65536), "rec"),
    ("rec_planes_to_rgb", 1, (3, 70000), (70000, 1), (1, 3), "rec"),
    ("rec_aos_to_soa_f32x17", 4, (4000, 17), (17, 1), (1, 4000), "rec"),
    ("rec_aos_to_soa_f16x6", 2, (3, 9000, 6), (54000, 6, 1), (54000, 1, 9000), "rec"),
    ("rec_aos_to_soa_u64x3", 8, (5000, 3), (3, 1), (1, 5000), "rec"),
    ("rec_aos_to_soa_f32x2_short", 4, (5, 2), (2, 1), (1, 8), "rec"),
    ("quad_aos_to_soa_f32x4", 4, (100000, 4), (4, 1), (1, 100000), "quad"),
    ("quad_aos_to_soa_f32x8_batched", 4, (3, 4096, 8), (32768, 8, 1), (32768, 1, 4096), "quad"),
    ("quad_aos_to_soa_f32x12_padded", 4, (2000, 12), (16, 1), (1, 2048), "quad"),
    ("quad_soa_to_aos_f32x8", 4, (8, 100000), (100000, 1), (1, 8), "quad"),
    ("quad_soa_to_aos_f32x12_batched", 4, (2, 12, 4096), (12 * 4096, 4096, 1), (12 * 4096, 1, 12), "quad"),
    ("copy_outer_perm", 4, (8, 64, 32), (32, 256, 1), (2048, 32, 1), "copy"),
    ("copy_identity", 2, (1000, 64), (64, 1), (64, 1), "copy"),
    ("copy_runs_of_8_bytes", 2, (40, 12), (12, 1), (480, 1), "copy"),
    ("copy_runs_of_4_bytes", 1, (3, 50, 4), (200, 4, 1), (4, 12, 1), "copy"),
    ("rec_unaligned_rows_dense_dst", 2, (130, 1000), (1000, 1), (1, 130), "rec"),
    ("etile_unaligned_rows_padded_dst", 2, (130, 1000), (1000, 1), (1, 131), "etile"),
    ("gather_no_unit_stride", 4, (16, 24), (48, 2), (24, 1), "gather"),
    ("gather_small_modes", 8, (3, 5, 7), (35, 7, 1), (1, 3, 15), "gather"),
    ("lds_broadcast_src", 4, (64, 32), (0, 1), (1, 64), "lds"),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: c[0])
def test_ragged_and_kernel_families(case):
    name, w, ext, ss, ds, kernel = case
    batch = 3 if kernel not in ("lds", "rec") else 1
    run_case(name, w, ext, ss, ds, seed=zlib.crc32(name.encode()) & 0xFFFF, expect_kernel=kernel, batch=batch)


@pytest.mark.parametrize("w,offs", [(4, (3, 0)), (4, (0, 5)), (2, (1, 7)), (16, (1, 1)), (1, (3, 9))])
def test_unaligned_offsets(w, offs):
    """Offsets that break 16-byte alignment fall back to narrower accesses."""
    ext = (4, 32) if w == 4 else (64, 48)
    ss = (ext[1], 1)
    ds = (1, ext[0])
    run_case(f"unaligned_w{w}_{offs}", w, ext, ss, ds, offs, batch=5, seed=w * 31 + offs[0])


def test_random_layouts():
    rng = np.random.default_rng(99)
    for t in range(24):
        rank = int(rng.integers(1, 5))
        w = int(rng.choice([1, 2, 4, 8, 16]))
        ext = [int(rng.integers(1, 9)) for _ in range(rank)]
        order = list(rng.permutation(rank))
        ds = [0] * rank
        acc = 1
        for ax in reversed(order):
            ds[ax] = acc
            acc *= ext[ax] + int(rng.integers(0, 2))
        ss = [int(rng.integers(0, 9)) for _ in range(rank)]
        offs = (int(rng.integers(0, 4)), int(rng.integers(0, 4)))
        run_case(f"random_{t}", w, ext, ss, ds, offs, batch=int(rng.integers(1, 4)), seed=t)


# ---------------------------------------------------------------------------
# in place, overlap, declines, empty


@pytest.mark.parametrize("w", [1, 2])
def test_inplace_sub_dword_sf_transpose(w):
    """1- and 2-byte SF tiles in place: each batch item is moved inside one
    wave-instruction by the quad kernel, reads before writes."""
    torch = _torch()
    print(f"\n[case] in-place SF transpose, w={w}, 2^16 tiles", flush=True)
    batch = 1 << 16
    x = make_input(40 + w, batch * 128 * w)
    ref = np.empty_like(x)
    oracle.permute(x, ref, w, (4, 32), (32, 1), (1, 4), (0, 0), batch)
    assert tpl.tpl_plan(w, (4, 32), (32, 1), (1, 4), batch=batch, geometry=tpl.TPL_GEOM_GFX950_INPLACE).kernel == "quad"
    buf = torch.from_numpy(x).cuda()
    tpl.permute(buf, buf, (4, 32), (32, 1), (1, 4), batch=batch, dtype_bytes=w)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), ref)


def test_inplace_sf_transpose():
    torch = _torch()
    wl = workloads.SF_BATCHED
    print("\n[case] inplace SF transpose, full size", flush=True)
    n = wl.elements * 4
    x = make_input(wl.seed, n, True)
    ref = np.empty_like(x)
    oracle.permute(x, ref, 4, wl.extents, wl.src_strides, wl.dst_strides, (0, 0), wl.batch)
    buf = torch.from_numpy(x).cuda()
    tpl.permute(buf, buf, wl.extents, wl.src_strides, wl.dst_strides, batch=wl.batch, dtype_bytes=4)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), ref)


def test_inplace_tile_move():
    torch = _torch()
    wl = workloads.scaled(workloads.TILE_128x64, batch=256)
    print("\n[case] inplace 128x64 fp16 tiles", flush=True)
    n = wl.elements * 2
    x = make_input(wl.seed, n)
    ref = np.empty_like(x)
    oracle.permute(x, ref, 2, wl.extents, wl.src_strides, wl.dst_strides, (0, 0), wl.batch)
    buf = torch.from_numpy(x).cuda()
    tpl.permute(buf, buf, wl.extents, wl.src_strides, wl.dst_strides, batch=wl.batch, dtype_bytes=2)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), ref)


def test_overlap_other_than_in_place_is_refused():
    torch = _torch()
    print("\n[case] partial overlap -> TPL_E_ALIAS, buffer untouched", flush=True)
    x = make_input(7, 16384 * 4)
    buf = torch.from_numpy(x).cuda()
    with pytest.raises(tpl.TplError) as e:
        # dst starts 64 elements into src
        tpl.permute(buf, buf, (4, 32), (32, 1), (1, 4), src_offset=0, dst_offset=64, batch=8, dtype_bytes=4)
    assert e.value.status == tpl.TPL_E_ALIAS
    # a non-square in-place transpose over several tiles moves data across units: refused too
    with pytest.raises(tpl.TplError) as e:
        tpl.permute(buf, buf, (64, 32), (32, 1), (1, 64), batch=2, dtype_bytes=8)
    assert e.value.status == tpl.TPL_E_ALIAS
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), x)


def test_inplace_single_tile_transpose():
    """A 64x64 fp32 transpose is one workgroup tile: it may run in place."""
    torch = _torch()
    print("\n[case] in-place 64x64 fp32 transpose (one tile)", flush=True)
    x = make_input(8, 64 * 64 * 4)
    ref = np.empty_like(x)
    oracle.permute(x, ref, 4, (64, 64), (64, 1), (1, 64))
    assert tpl.tpl_plan(4, (64, 64), (64, 1), (1, 64)).kernel == "lds"
    buf = torch.from_numpy(x).cuda()
    tpl.permute(buf, buf, (64, 64), (64, 1), (1, 64), dtype_bytes=4)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), ref)


@pytest.mark.parametrize("w,ext,ss,ds,status", [
    (3, (4, 32), (32, 1), (1, 4), tpl.TPL_E_DTYPE_WIDTH),
    (4, (4, 32), (32, 1), (1, 2), tpl.TPL_E_LAYOUT),
    (4, (4, 32), (32, 1), (0, 4), tpl.TPL_E_LAYOUT),
])
def test_declined_call_leaves_dst_untouched(w, ext, ss, ds, status):
    torch = _torch()
    print(f"\n[case] decline status {status}", flush=True)
    s = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    d = torch.full((4096,), SENTINEL, dtype=torch.uint8, device="cuda")
    st = tpl.tpl_permute(s.data_ptr(), d.data_ptr(), w, ext, ss, ds, (0, 0), 1, 0)
    assert st == status
    torch.cuda.synchronize()
    assert bool((d == SENTINEL).all())


def test_empty_launches_nothing():
    torch = _torch()
    print("\n[case] empty extents and batch 0", flush=True)
    s = torch.zeros(512, dtype=torch.uint8, device="cuda")
    d = torch.full((512,), SENTINEL, dtype=torch.uint8, device="cuda")
    tpl.permute(d, s, (0, 32), (32, 1), (1, 4), dtype_bytes=4)
    tpl.permute(d, s, (4, 32), (32, 1), (1, 4), batch=0, dtype_bytes=4)
    torch.cuda.synchronize()
    assert bool((d == SENTINEL).all())


def test_repeatable():
    torch = _torch()
    print("\n[case] the same call twice gives identical bytes", flush=True)
    wl = workloads.scaled(workloads.TILE_128x64, batch=512)
    x = torch.from_numpy(make_input(3, wl.elements * 2)).cuda()
    outs = []
    for _ in range(2):
        d = torch.full((wl.elements * 2,), SENTINEL, dtype=torch.uint8, device="cuda")
        tpl.permute(d, x, wl.extents, wl.src_strides, wl.dst_strides, batch=wl.batch, dtype_bytes=2)
        outs.append(d)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


BIG_CASES = [
    # name, w, extents, src strides, dst strides, batch, kernel
    ("lds_u8_axes021", 1, (48, 65536, 704), (704 * 65536, 704, 1), (704 * 65536, 1, 65536), 1, "lds"),
    ("quad_u8_sf", 1, (4, 32), (32, 1), (1, 4), 1 << 24, "quad"),
    ("rec_rgb_to_planes", 1, (1 << 30, 3), (3, 1), (1, 1 << 30), 1, "rec"),
    ("rec_planes_to_rgb", 1, (3, 3 << 28), (3 << 28, 1), (1, 3), 1, "rec"),
    ("copy_u8_row_blocks", 1, (2, 1024, 1 << 20), (1 << 30, 1 << 20, 1), (1 << 20, 1 << 21, 1), 1, "copy"),
    ("gather_u8_stride2", 1, (1 << 31,), (2,), (1,), 1, "gather"),
]


def oracle_threads(x, ref, w, ext, ss, ds, batch):
    """The C oracle over the whole layout, run on slices of the outermost
    index in host threads (the oracle's ctypes call releases the GIL).  By the
    address rule, batch items [a, b) start a * span further on each side, and
    with one item, rows [a, b) of the first mode start a * stride further."""
    import concurrent.futures as cf
    import os
    span_s, span_d = cosize(ext, ss), cosize(ext, ds)
    n = batch if batch > 1 else ext[0]
    threads = max(1, min(16, os.cpu_count() or 1, n))
    cuts = [n * i // threads for i in range(threads + 1)]

    def one(a, b):
        if batch > 1:
            oracle.permute(x, ref, w, ext, ss, ds, (a * span_s, a * span_d), b - a)
        else:
            oracle.permute(x, ref, w, (b - a,) + tuple(ext[1:]), ss, ds, (a * ss[0], a * ds[0]), 1)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda ab: one(*ab), [(a, b) for a, b in zip(cuts, cuts[1:]) if b > a]))
    return ref


def check_full(name, got, ref):
    if not np.array_equal(got, ref):
        diff = np.flatnonzero(got != ref)
        raise AssertionError(f"{name}: {diff.size} bytes differ; first at byte {diff[0]}")


@pytest.mark.parametrize("case", BIG_CASES, ids=lambda c: c[0])
def test_big_index_paths(case):
    """At least 2^31 elements (the kernels' 64-bit index instances): the whole
    result against the oracle's, byte for byte, with the destination's
    sentinel bytes on both sides."""
    torch = _torch()
    name, w, ext, ss, ds, batch, kernel = case
    n = batch
    for e in ext:
        n *= e
    assert n >= 1 << 31
    plan = tpl.tpl_plan(w, ext, ss, ds, batch=batch)
    assert plan.kernel == kernel, plan
    print(f"\n[case] big index path {name}: {n} elements, kernel {plan.kernel}", flush=True)
    nbs, nbd = batch * cosize(ext, ss) * w, batch * cosize(ext, ds) * w
    gen = torch.Generator("cuda").manual_seed(5)
    x = torch.randint(0, 256, (nbs,), dtype=torch.uint8, device="cuda", generator=gen)
    d = torch.full((nbd,), SENTINEL, dtype=torch.uint8, device="cuda")
    tpl.permute(d, x, ext, ss, ds, batch=batch, dtype_bytes=w)
    torch.cuda.synchronize()
    xh = x.cpu().numpy()
    del x
    got = d.cpu().numpy()
    del d
    torch.cuda.empty_cache()
    ref = oracle_threads(xh, np.full(nbd, SENTINEL, dtype=np.uint8), w, ext, ss, ds, batch)
    check_full(name, got, ref)


BIG_ETILE = [
    # name, w, extents, src strides, dst strides, src swizzle: the element
    # tiles' 64-bit instances (tall vector form, shifted and aligned
    # destination rows; the element form)
    ("etile_tall_u8_dst_pitch_46403", 1, (46400, 46400), (46400, 1), (1, 46403), None),
    ("etile_tall_bf16_src_pitch_65601", 2, (32800, 65600), (65601, 1), (1, 32800), None),
    ("etile_element_u8_src_swizzle_203", 1, (46400, 46400), (46400, 1), (1, 46400), (2, 0, 3)),
]


@pytest.mark.parametrize("case", BIG_ETILE, ids=lambda c: c[0])
def test_big_element_tiles(case):
    """Element tiles over at least 2^31 elements: the whole result against
    the oracle's, byte for byte, sentinel bytes kept."""
    torch = _torch()
    name, w, ext, ss, ds, zs = case
    assert ext[0] * ext[1] >= 1 << 31
    plan = tpl.tpl_plan(w, ext, ss, ds, src_swizzle=zs)
    assert plan.kernel == "etile", plan
    print(f"\n[case] big element tiles {name}: tile {tuple(plan.tile)}", flush=True)
    nbs, nbd = cosize(ext, ss) * w, cosize(ext, ds) * w
    gen = torch.Generator("cuda").manual_seed(8)
    x = torch.randint(0, 256, (nbs,), dtype=torch.uint8, device="cuda", generator=gen)
    d = torch.full((nbd,), SENTINEL, dtype=torch.uint8, device="cuda")
    tpl.permute(d, x, ext, ss, ds, dtype_bytes=w, src_swizzle=zs)
    torch.cuda.synchronize()
    xh = x.cpu().numpy()
    del x
    got = d.cpu().numpy()
    del d
    torch.cuda.empty_cache()
    ref = np.full(nbd, SENTINEL, dtype=np.uint8)
    if zs is None:
        ref = oracle_threads(xh, ref, w, ext, ss, ds, 1)
    else:
        oracle.permute(xh, ref, w, ext, ss, ds, (0, 0), 1, zs, None)
    check_full(name, got, ref)


def test_big_in_place_transpose():
    """A 65536 x 65536 byte matrix (2^32 elements) transposed in place by the
    tile-pair swap kernel's 64-bit instance, against the oracle's
    out-of-place result on a copy of the input."""
    torch = _torch()
    ext, ss, ds = (65536, 65536), (65536, 1), (1, 65536)
    plan = tpl.tpl_plan(1, ext, ss, ds, geometry=tpl.TPL_GEOM_GFX950_INPLACE)
    assert plan.kernel == "swap", plan
    print("\n[case] big in-place transpose 65536x65536 u8, kernel swap", flush=True)
    gen = torch.Generator("cuda").manual_seed(6)
    buf = torch.randint(0, 256, (1 << 32,), dtype=torch.uint8, device="cuda", generator=gen)
    x0 = buf.cpu().numpy()
    tpl.permute(buf, buf, ext, ss, ds, dtype_bytes=1)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    del buf
    torch.cuda.empty_cache()
    ref = oracle_threads(x0, np.full(1 << 32, SENTINEL, dtype=np.uint8), 1, ext, ss, ds, 1)
    check_full("big in-place transpose", got, ref)


# ---------------------------------------------------------------------------
# tpl.copy_view: layouts taken from torch views


def _storage_bytes(t):
    import torch
    return t.contiguous().view(torch.uint8).reshape(-1).cpu().numpy().copy()


def _view_case(name, dst_base, dst, src_base, src):
    torch = _torch()
    print(f"\n[case] copy_view {name}: shape={tuple(src.shape)} src strides={src.stride()} "
          f"dst strides={dst.stride()}", flush=True)
    w = src.element_size()
    dims = [i for i, e in enumerate(src.shape) if e != 1]
    ext = tuple(src.shape[i] for i in dims)
    ss = tuple(src.stride(i) for i in dims)
    ds = tuple(dst.stride(i) for i in dims)
    same = src_base.data_ptr() == dst_base.data_ptr()
    xs = _storage_bytes(src_base)
    ref = xs.copy() if same else _storage_bytes(dst_base)
    oracle.permute(xs, ref, w, ext, ss, ds, (src.storage_offset(), dst.storage_offset()), 1)
    tpl.copy_view(dst, src)
    torch.cuda.synchronize()
    got = _storage_bytes(dst_base)
    assert np.array_equal(got, ref), f"{name}: {int(np.count_nonzero(got != ref))} bytes differ"


def test_copy_view_matches_oracle():
    torch = _torch()
    g = torch.Generator("cuda").manual_seed(21)

    def nbytes(shape, dtype):
        return int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()

    def rnd(shape, dtype):   # random bit patterns of any dtype
        return torch.randint(0, 256, (nbytes(shape, dtype),), dtype=torch.uint8, device="cuda",
                             generator=g).view(dtype).reshape(shape)

    def filled(shape, dtype):   # sentinel bytes
        return torch.full((nbytes(shape, dtype),), SENTINEL, dtype=torch.uint8, device="cuda").view(dtype).reshape(shape)

    # a permuted source into a contiguous destination (fp32)
    a = rnd((64, 128, 32), torch.float32)
    d = filled((32, 64, 128), torch.float32)
    _view_case("permuted_src", d, d, a, a.permute(2, 0, 1))
    # contiguous bf16 source into a transposed destination view
    a = rnd((96, 200), torch.bfloat16)
    db = filled((200, 96), torch.bfloat16)
    _view_case("transposed_dst", db, db.t(), a, a)
    # a column slice of bytes into a transposed destination
    a = rnd((128, 300), torch.uint8)
    db = filled((256, 128), torch.uint8)
    _view_case("sliced_src", db, db.t(), a, a[:, 7:263])
    # a broadcast (stride-0) fp16 row into a contiguous block
    a = rnd((1, 64), torch.float16)
    d = filled((48, 64), torch.float16)
    _view_case("broadcast_src", d, d, a, a.expand(48, 64))
    # a strided sub-view of 8-byte elements into a transposed destination
    a = rnd((40, 3, 17), torch.float64)
    db = filled((17, 40), torch.float64)
    _view_case("strided_subview", db, db.t(), a, a[:, 1, :])
    # a square matrix onto its own transpose: in place
    a = rnd((512, 512), torch.float32)
    _view_case("in_place_transpose", a, a, a, a.t())


# ---------------------------------------------------------------------------
# Element tiles: 2-D transposes that 16-byte vectors cannot serve (odd row
# pitches, element offsets, small swizzle granules), tiled through LDS: plain
# operands of 1-4 bytes as the aligned 16-byte chunks covering each row piece
# (the vector form), 8-byte elements and swizzled operands one element per
# access.

ETILE = [
    # name, w, extents, src strides, dst strides, element offsets, batch, src swizzle, dst swizzle
    ("u8_odd_pitches", 1, (300, 260), (261, 1), (1, 301), (0, 0), 1, None, None),
    ("bf16_odd_pitches_ragged", 2, (257, 513), (515, 1), (1, 257), (0, 0), 1, None, None),
    ("f32_offsets_batch", 4, (200, 300), (301, 1), (1, 200), (3, 1), 3, None, None),
    ("f64_odd_pitches", 8, (100, 90), (91, 1), (1, 101), (0, 0), 1, None, None),
    ("u16_src_offset_odd", 2, (128, 256), (256, 1), (1, 128), (1, 0), 2, None, None),
    ("f32_into_8B_granule_swizzle", 4, (64, 96), (96, 1), (1, 64), (0, 0), 2, None, (3, 1, 3)),
    ("u8_from_2B_granule_swizzle", 1, (96, 160), (160, 1), (1, 96), (0, 0), 1, (2, 1, 4), None),
    ("below_one_tile", 4, (12, 20), (21, 1), (1, 13), (0, 0), 5, None, None),
    # vector form: destination rows not on 16 bytes (partial first and last chunks)
    ("u8_dst_pitch_odd_only", 1, (300, 256), (256, 1), (1, 301), (0, 0), 1, None, None),
    ("bf16_dst_pitch_odd_batch", 2, (260, 200), (200, 1), (1, 263), (0, 0), 2, None, None),
    ("f32_dst_offset_only", 4, (256, 96), (96, 1), (1, 256), (0, 1), 1, None, None),
    # every lead on both sides, offsets, ragged in both directions
    ("u8_every_lead_both_sides", 1, (515, 333), (337, 1), (1, 519), (7, 9), 1, None, None),
    ("bf16_one_past_a_tile", 2, (129, 65), (67, 1), (1, 131), (1, 1), 1, None, None),
    ("f32_many_tiles_odd", 4, (1000, 700), (701, 1), (1, 1003), (0, 0), 1, None, None),
]


@pytest.mark.parametrize("case", ETILE, ids=lambda c: c[0])
def test_element_tiles_match_oracle(case):
    name, w, ext, ss, ds, offs, batch, zs, zd = case
    run_case(f"etile_{name}", w, ext, ss, ds, offs, batch, seed=zlib.crc32(name.encode()) & 0xFFFF,
             expect_kernel="etile", zs=zs, zd=zd)


def test_element_tiles_full_size():
    """A 16384 x 16384 bf16 transpose with source rows 16385 elements apart
    (no 16-byte alignment on any row but the first): the whole result
    against the oracle's."""
    torch = _torch()
    ext, ss, ds = (16384, 16384), (16385, 1), (1, 16384)
    plan = tpl.tpl_plan(2, ext, ss, ds)
    assert plan.kernel == "etile", plan
    print("\n[case] element tiles 16384^2 bf16, source pitch 16385", flush=True)
    nbs, nbd = cosize(ext, ss) * 2, cosize(ext, ds) * 2
    gen = torch.Generator("cuda").manual_seed(9)
    x = torch.randint(0, 256, (nbs,), dtype=torch.uint8, device="cuda", generator=gen)
    d = torch.full((nbd,), SENTINEL, dtype=torch.uint8, device="cuda")
    tpl.permute(d, x, ext, ss, ds, dtype_bytes=2)
    torch.cuda.synchronize()
    ref = oracle_threads(x.cpu().numpy(), np.full(nbd, SENTINEL, dtype=np.uint8), 2, ext, ss, ds, 1)
    check_full("element tiles 16384^2", d.cpu().numpy(), ref)


ETILE_LARGE = [
    # (name, w, extents, src strides, dst strides, src swizzle): launches of
    # 8192 tiles or more (the three-per-CU reserve of the vector form with
    # aligned destination rows), the shifted form at that size, and the
    # element form with its batched loads
    ("u8_16384sq_src_pitch_16387", 1, (16384, 16384), (16387, 1), (1, 16384), None),
    ("f32_8192sq_src_pitch_8193", 4, (8192, 8192), (8193, 1), (1, 8192), None),
    ("bf16_16384sq_dst_pitch_16385", 2, (16384, 16384), (16384, 1), (1, 16385), None),
    ("u8_8192sq_dst_pitch_8195", 1, (8192, 8192), (8192, 1), (1, 8195), None),
    # tall tiles: the shifted form from 2048 tall tiles (bf16, u8 above), a
    # ragged one, and bf16 with aligned destination rows from 16384
    ("bf16_8192sq_dst_pitch_8193", 2, (8192, 8192), (8192, 1), (1, 8193), None),
    ("bf16_8000x8100_dst_pitch_8003", 2, (8000, 8100), (8100, 1), (1, 8003), None),
    ("u8_4x2048x8192_dst_pitch_2051", 1, (4, 2048, 8192), (2048 * 8192, 8192, 1), (8192 * 2051, 1, 2051), None),
    ("bf16_16384sq_src_pitch_16385", 2, (16384, 16384), (16385, 1), (1, 16384), None),
    ("f64_4096sq_src_pitch_4097", 8, (4096, 4096), (4097, 1), (1, 4096), None),
    ("bf16_4096sq_src_swizzle_323", 2, (4096, 4096), (4096, 1), (1, 4096), (3, 2, 3)),
]


@pytest.mark.parametrize("case", ETILE_LARGE, ids=lambda c: c[0])
def test_element_tiles_large(case):
    """Element tiles at sizes that take the launch-size dependent choices:
    the whole result against the oracle's."""
    torch = _torch()
    name, w, ext, ss, ds, zs = case
    plan = tpl.tpl_plan(w, ext, ss, ds, src_swizzle=zs)
    assert plan.kernel == "etile", plan
    print(f"\n[case] element tiles {name}", flush=True)
    nbs, nbd = cosize(ext, ss) * w, cosize(ext, ds) * w
    gen = torch.Generator("cuda").manual_seed(11)
    x = torch.randint(0, 256, (nbs,), dtype=torch.uint8, device="cuda", generator=gen)
    d = torch.full((nbd,), SENTINEL, dtype=torch.uint8, device="cuda")
    tpl.permute(d, x, ext, ss, ds, dtype_bytes=w, src_swizzle=zs)
    torch.cuda.synchronize()
    ref = np.full(nbd, SENTINEL, dtype=np.uint8)
    if zs is None:
        ref = oracle_threads(x.cpu().numpy(), ref, w, ext, ss, ds, 1)
    else:
        oracle.permute(x.cpu().numpy(), ref, w, ext, ss, ds, (0, 0), 1, zs, None)
    check_full(name, d.cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# The largest rank the ABI takes: 8 modes, permuted axis orders.

def _row_major_order(ext, order):
    st = [0] * len(ext)
    acc = 1
    for ax in reversed(order):
        st[ax] = acc
        acc *= ext[ax]
    return tuple(st)


RANK8 = [
    ("rank8_u32_scrambled", 4, (2, 3, 2, 4, 2, 3, 2, 5), (7, 0, 5, 2, 3, 6, 1, 4), 1),
    ("rank8_u16_last_axis_kept", 2, (2, 2, 3, 2, 2, 3, 4, 64), (1, 0, 3, 2, 5, 4, 6, 7), 3),
    ("rank8_u8_reversed", 1, (3, 2, 2, 3, 2, 2, 5, 32), (7, 6, 5, 4, 3, 2, 1, 0), 2),
]


@pytest.mark.parametrize("case", RANK8, ids=lambda c: c[0])
def test_rank8_permutations_match_oracle(case):
    name, w, ext, order, batch = case
    ss = _row_major_order(ext, list(range(8)))
    ds = _row_major_order(ext, list(order))
    run_case(name, w, ext, ss, ds, (0, 0), batch, seed=zlib.crc32(name.encode()) & 0xFFFF)


# ---------------------------------------------------------------------------
# Every tile shape the tiled transpose instantiates, picked by extents just
# past the shape (ragged edges on both modes), as one item and as two items
# of a batch mode.  Shapes carry their chunks per thread; how a case reaches
# its shape:
#   strided    -- the width's 32 KiB shape run at two workgroups per CU (tiles
#                 strided on both sides, source rows shorter than 4x the
#                 destination's);
#   short_dst  -- the source-contiguous extent at least 4x the destination-
#                 contiguous one;
#   dst_block  -- destination rows of exactly the tile's extent, adjacent, so a
#                 tile's destination is one block and the general list applies;
#   general    -- extents too small for the strided shape.

LDS_SHAPES = [
    (1, 128, 128, 4, "strided"), (1, 128, 128, 2, "dst_block"), (1, 64, 128, 2, "general"),
    (2, 256, 64, 4, "strided"), (2, 256, 64, 2, "dst_block"), (2, 128, 64, 2, "general"), (2, 32, 64, 2, "general"),
    (2, 128, 128, 4, "short_dst"),
    (4, 128, 64, 4, "strided"), (4, 64, 64, 2, "general"), (4, 32, 32, 2, "general"), (4, 32, 256, 2, "short_dst"),
    (8, 64, 64, 4, "strided"), (8, 32, 64, 2, "general"), (8, 16, 32, 2, "general"),
    (16, 64, 16, 2, "strided"), (16, 64, 16, 2, "dst_block"), (16, 16, 64, 2, "general"), (16, 16, 16, 2, "general"),
]


def _shape_case(w, tb, ta, mode):
    eb, ea = tb + 3, ta + 5
    if mode == "short_dst":
        ea = max(ea, 4 * eb)
    if mode == "dst_block":
        eb = tb
    pa = -(-ea * w // 16) * 16 // w    # rows padded to whole 16-byte chunks
    pb = eb if mode == "dst_block" else -(-eb * w // 16) * 16 // w
    return eb, ea, pa, pb


@pytest.mark.parametrize("shape", LDS_SHAPES, ids=lambda s: f"w{s[0]}_{s[1]}x{s[2]}_cpt{s[3]}_{s[4]}")
def test_every_lds_tile_shape(shape):
    w, tb, ta, cpt, mode = shape
    eb, ea, pa, pb = _shape_case(w, tb, ta, mode)
    ext, ss, ds = (eb, ea), (pa, 1), (1, pb)
    p = tpl.tpl_plan(w, ext, ss, ds)
    assert p.kernel == "lds" and tuple(p.tile) == (tb, ta) and p.chunks_per_thread == cpt, p
    run_case(f"lds_shape_w{w}_{tb}x{ta}_cpt{cpt}_{mode}", w, ext, ss, ds, seed=tb * 7 + ta + cpt)
    # two items 16-byte aligned apart: one batch mode
    item_s, item_d = eb * pa + 16 // min(w, 16), ea * pb + 16 // min(w, 16)
    ext3, ss3, ds3 = (2, eb, ea), (item_s, pa, 1), (item_d, 1, pb)
    p3 = tpl.tpl_plan(w, ext3, ss3, ds3)
    assert p3.kernel == "lds" and tuple(p3.tile) == (tb, ta) and p3.chunks_per_thread == cpt, p3
    run_case(f"lds_shape_w{w}_{tb}x{ta}_cpt{cpt}_{mode}_two_items", w, ext3, ss3, ds3, seed=tb * 7 + ta + cpt + 1)
