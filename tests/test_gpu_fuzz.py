"""Randomised GPU parity: tensor permutations of random shapes, widths,
offsets, batches and swizzles, sized so that every kernel family is reached,
each case checked byte for byte against the oracle.  Also: capture in a HIP
graph and replay, and two streams at once."""

from __future__ import annotations

import collections
import os

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl
from tests.test_gpu_parity import run_case, make_input, sizes, SENTINEL
from tests.test_gpu_inplace import run_inplace

pytestmark = pytest.mark.gpu

# TPL_FUZZ_SCALE=k runs k times as many random cases (the same seeds, longer
# sequences); 1 by default.
SCALE = max(1, int(os.environ.get("TPL_FUZZ_SCALE", "1")))


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def random_case(rng, aligned=False):
    """aligned: 16-byte aligned rows and offsets and swizzle granules of at
    least 16 bytes, so that the vector kernels take the case."""
    rank = int(rng.integers(2, 5))
    w = int(rng.choice([1, 2, 4, 8, 16]))
    # extents: mostly tile-friendly sizes, some ragged
    pool = [4, 16, 32, 64, 96, 128] if aligned else [1, 3, 4, 16, 32, 48, 64, 96, 128, 130, 256]
    ext = [int(rng.choice(pool)) for _ in range(rank)]
    while int(np.prod(ext)) * w > (4 << 20):
        ext[int(np.argmax(ext))] //= 2
    ext = [max(1, e) for e in ext]
    # source: row-major, maybe with padded rows; destination: row-major of a
    # random axis order, maybe padded
    def row_major(order, pad):
        st = [0] * rank
        acc = 1
        for ax in reversed(order):
            st[ax] = acc
            acc *= ext[ax] + (pad if ax == order[-1] else 0)
        return st
    ss = row_major(list(range(rank)), int(rng.choice([0, 0, 16] if aligned else [0, 0, 16, 5])))
    ds = row_major(list(rng.permutation(rank)), int(rng.choice([0, 0, 16])))
    offs = (int(rng.choice([0, 0, 0, 16] if aligned else [0, 0, 0, 16, 3])),
            int(rng.choice([0, 0, 0, 32] if aligned else [0, 0, 0, 32, 5])))
    batch = int(rng.choice([1, 1, 2, 3]))
    lw = {1: 0, 2: 1, 4: 2, 8: 3, 16: 4}[w]

    def swz():
        if rng.random() < 0.7:
            return None
        bits = int(rng.integers(1, 4))
        base = int(rng.integers(max(0, 4 - lw), 6)) if aligned else int(rng.integers(0, 4))
        return (bits, base, int(rng.integers(bits, 6)))
    return w, ext, ss, ds, offs, batch, swz(), swz()


def test_random_permutations_match_oracle():
    rng = np.random.default_rng(20261202)
    kernels = collections.Counter()
    for t in range(80 * SCALE):
        w, ext, ss, ds, offs, batch, zs, zd = random_case(rng, aligned=t % 2 == 1)
        p = tpl.tpl_plan(w, ext, ss, ds, offs, batch, src_swizzle=zs, dst_swizzle=zd)
        assert p.ok, (t, p)
        kernels[p.kernel] += 1
        run_case(f"fuzz_{t}", w, ext, ss, ds, offs, batch, seed=t, zs=zs, zd=zd)
    print("kernel mix:", dict(kernels), flush=True)
    assert {"lds", "gather", "copy", "quad", "etile"} <= set(kernels)


def record_case(rng):
    """Records of F fields (2..20) to one row per field, or back; rows mostly
    padded to whole 16-byte pieces, some ragged or misaligned."""
    w = int(rng.choice([1, 2, 4, 8, 16]))
    F = int(rng.integers(2, 21))
    while F * w > 1024:
        F //= 2
    N = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 6000)), int(rng.integers(64, 6000))]))
    align = max(1, 16 // w)
    N = N if rng.random() < 0.3 else -(-N // align) * align
    pad = int(rng.choice([0, 0, align, 3]))
    rowlen = N + pad
    batch = int(rng.choice([1, 1, 2, 3]))
    if rng.random() < 0.5:
        ext, ss, ds = (N, F), (F, 1), (1, rowlen)
    else:
        ext, ss, ds = (F, N), (rowlen, 1), (1, F)
    offs = (int(rng.choice([0, 0, 0, align, 1])), int(rng.choice([0, 0, 0, 2 * align, 2])))
    return w, ext, ss, ds, offs, batch


def random_unaligned_transpose(rng):
    """A 2-D transpose (plus batch) whose rows miss 16-byte alignment on one
    side or both: random width, extents, row pitches, element offsets,
    batch with or without gaps between items."""
    w = int(rng.choice([1, 2, 4, 8]))
    e_b = int(rng.integers(8, 700))
    e_a = int(rng.integers(8, 700))
    while e_a * e_b * w > (2 << 20):
        e_a, e_b = max(8, e_a // 2), max(8, e_b // 2)
    ps = e_a + int(rng.choice([0, 1, 2, 3, 5, 7, 16, 17]))
    pd = e_b + int(rng.choice([0, 1, 3, 8, 9, 15]))
    offs = (int(rng.integers(0, 20)), int(rng.choice([0, 0, 1, 4, 13])))
    batch = int(rng.choice([1, 1, 2, 3]))
    ext, ss, ds = (e_b, e_a), (ps, 1), (1, pd)
    if batch > 1 and rng.random() < 0.5:
        # items further apart than their span
        span_s, span_d = (e_b - 1) * ps + e_a, (e_a - 1) * pd + e_b
        gs, gd = int(rng.integers(0, 40)), int(rng.integers(0, 40))
        ext, ss, ds = (batch, e_b, e_a), (span_s + gs, ps, 1), (span_d + gd, 1, pd)
        batch = 1
    return w, ext, ss, ds, offs, batch


def test_random_unaligned_transposes_match_oracle():
    """The element-tile kernel's two forms (16-byte chunks for 1-4 byte
    elements, one element per access for 8-byte ones) on random unaligned
    layouts, byte for byte against the oracle."""
    rng = np.random.default_rng(1202)
    kernels = collections.Counter()
    for t in range(60 * SCALE):
        w, ext, ss, ds, offs, batch = random_unaligned_transpose(rng)
        p = tpl.tpl_plan(w, ext, ss, ds, offs, batch)
        assert p.ok, (t, p)
        kernels[(p.kernel, w)] += 1
        run_case(f"unaligned_{t}", w, ext, ss, ds, offs, batch, seed=1000 + t)
    print("kernel mix:", dict(kernels), flush=True)
    assert sum(n for (k, w), n in kernels.items() if k == "etile" and w <= 4) >= 30 * SCALE


def test_random_tall_element_tiles_match_oracle():
    """Random unaligned transposes of 1- and 2-byte elements large enough for
    the tall element tiles (unaligned destination rows, at least 2048 tall
    tiles: 32-80 MiB each way), byte for byte against the oracle."""
    rng = np.random.default_rng(2048)
    done = 0
    while done < 6 * SCALE:
        w = int(rng.choice([1, 2]))
        eb, ea = int(rng.integers(2000, 9000)), int(rng.integers(2000, 9000))
        tall_tb, tall_ta = (256, 128) if w == 1 else (256, 64)
        if -(-eb // tall_tb) * -(-ea // tall_ta) < 2048 or eb * ea * w > (80 << 20):
            continue
        ps = ea + int(rng.integers(0, 9))
        pd = eb + int(rng.integers(1, 16))
        offs = (int(rng.integers(0, 8)), int(rng.integers(0, 8)))
        if (pd * w) % 16 == 0 and (offs[1] * w) % 16 == 0:
            continue
        p = tpl.tpl_plan(w, (eb, ea), (ps, 1), (1, pd), offs, 1)
        assert p.ok and p.kernel == "etile" and tuple(p.tile) == (tall_tb, tall_ta), p
        run_case(f"tall_{done}", w, (eb, ea), (ps, 1), (1, pd), offs, 1, seed=3000 + done)
        done += 1


def test_random_degenerate_layouts_match_oracle():
    """Source layouts the definition allows but a permutation never has:
    zero strides (broadcast reads), strides smaller than the inner span
    (overlapping reads), size-1 modes; the destination a one-to-one layout
    (a permuted row-major order, sometimes padded); widths 1-16, offsets and
    batches.  Byte for byte against the oracle."""
    rng = np.random.default_rng(31)
    kernels = collections.Counter()
    done = 0
    while done < 40 * SCALE:
        w = int(rng.choice([1, 2, 4, 8, 16]))
        rank = int(rng.integers(1, 7))
        ext = [int(rng.choice([1, 2, 3, 4, 7, 8, 16, 32, 33, 64])) for _ in range(rank)]
        n = int(np.prod(ext))
        if n > 1 << 17:
            continue
        order = list(rng.permutation(rank))
        ds, acc = [0] * rank, 1
        for ax in reversed(order):
            ds[ax] = acc
            acc *= ext[ax] + int(rng.choice([0, 0, 1, 5]))
        ss = [int(rng.choice([0, 0, 1, 2, 3, 17, 64, 1000])) for _ in range(rank)]
        offs = (int(rng.integers(0, 9)), int(rng.integers(0, 9)))
        batch = int(rng.choice([1, 1, 2, 3]))
        p = tpl.tpl_plan(w, ext, ss, ds, offs, batch)
        assert p.ok, (ext, ss, ds, p)
        kernels[p.kernel] += 1
        run_case(f"degenerate_{done}", w, ext, ss, ds, offs, batch, seed=4000 + done)
        done += 1
    print("kernel mix:", dict(kernels), flush=True)


def test_random_record_layouts_match_oracle():
    rng = np.random.default_rng(7)
    kernels = collections.Counter()
    for t in range(60 * SCALE):
        w, ext, ss, ds, offs, batch = record_case(rng)
        p = tpl.tpl_plan(w, ext, ss, ds, offs, batch)
        assert p.ok, (t, p)
        kernels[p.kernel] += 1
        run_case(f"records_{t}", w, ext, ss, ds, offs, batch, seed=100 + t)
    print("kernel mix:", dict(kernels), flush=True)
    assert kernels["rec"] >= 10 * SCALE


def test_random_inplace_transposes_match_oracle():
    """Square transposes in place: widths, sizes from one tile to eleven
    8 x 8-tile blocks per side, padded or unaligned pitches, batches and
    offsets."""
    rng = np.random.default_rng(8)
    kernels = collections.Counter()
    for t in range(40 * SCALE):
        w = int(rng.choice([1, 2, 4, 8, 16]))
        n = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 900)),
                            int(rng.integers(900, 3000 if w <= 2 else 1500))]))
        pitch = n + int(rng.choice([0, 0, 0, 3, 16]))
        batch = int(rng.choice([1, 1, 2]))
        gap = int(rng.choice([0, 8])) if batch > 1 else 0
        offset = int(rng.choice([0, 0, 16, 1]))
        item = n * pitch + gap
        ext = (batch, n, n) if batch > 1 else (n, n)
        ss = (item, pitch, 1) if batch > 1 else (pitch, 1)
        ds = (item, 1, pitch) if batch > 1 else (1, pitch)
        p = tpl.tpl_plan(w, ext, ss, ds, (offset, offset), 1, geometry=tpl.TPL_GEOM_GFX950_INPLACE)
        assert p.ok, (t, p)
        kernels[p.kernel] += 1
        run_inplace(f"inplace_{t}", w, n, pitch, batch, gap, offset, seed=200 + t, expect_kernel=p.kernel)
    print("kernel mix:", dict(kernels), flush=True)
    assert kernels["swap"] >= 25 * SCALE


def test_graph_capture_and_replay():
    """The permute captured into a HIP graph (no memset or host sync in the
    path), replayed three times on new inputs with eager work in between:
    every replay equals the oracle."""
    torch = _torch()
    print("\n[case] graph capture: fp16 128x64 tiles x 512 and SF x 4096", flush=True)
    t_ext, t_ss, t_ds, t_b = (128, 64), (64, 1), (1, 128), 512
    f_ext, f_ss, f_ds, f_b = (4, 32), (32, 1), (1, 4), 4096
    a = torch.empty(t_b * 128 * 64 * 2, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    c = torch.empty(f_b * 128 * 4, dtype=torch.uint8, device="cuda")
    d = torch.empty_like(c)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        # one eager call first: plans are made outside the capture
        tpl.permute(b, a, t_ext, t_ss, t_ds, batch=t_b, dtype_bytes=2)
        tpl.permute(d, c, f_ext, f_ss, f_ds, batch=f_b, dtype_bytes=4)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        tpl.permute(b, a, t_ext, t_ss, t_ds, batch=t_b, dtype_bytes=2)
        tpl.permute(d, c, f_ext, f_ss, f_ds, batch=f_b, dtype_bytes=4)
    for rep in range(3):
        xa = synth.random_bytes(100 + rep, a.numel()).copy()
        xc = synth.random_bytes(200 + rep, c.numel()).copy()
        a.copy_(torch.from_numpy(xa))
        c.copy_(torch.from_numpy(xc))
        b.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rb = np.empty_like(xa)
        oracle.permute(xa, rb, 2, t_ext, t_ss, t_ds, (0, 0), t_b)
        rd = np.empty_like(xc)
        oracle.permute(xc, rd, 4, f_ext, f_ss, f_ds, (0, 0), f_b)
        assert np.array_equal(b.cpu().numpy(), rb), rep
        assert np.array_equal(d.cpu().numpy(), rd), rep


def test_two_streams_at_once():
    torch = _torch()
    print("\n[case] two streams: bf16 2048^2 transpose and u8 (64,128,32,32) axes (0,2,3,1)", flush=True)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    n = 2048
    x1 = synth.random_bytes(301, n * n * 2).copy()
    e2, ss2, ds2 = (64, 128, 32, 32), (131072, 1024, 32, 1), (131072, 1, 4096, 128)
    x2 = synth.random_bytes(302, 64 * 128 * 32 * 32).copy()
    a1 = torch.from_numpy(x1).cuda()
    a2 = torch.from_numpy(x2).cuda()
    b1, b2 = torch.empty_like(a1), torch.empty_like(a2)
    torch.cuda.synchronize()
    for _ in range(4):
        with torch.cuda.stream(s1):
            tpl.permute(b1, a1, (n, n), (n, 1), (1, n), dtype_bytes=2)
        with torch.cuda.stream(s2):
            tpl.permute(b2, a2, e2, ss2, ds2, dtype_bytes=1)
    torch.cuda.synchronize()
    r1 = np.empty_like(x1)
    oracle.permute(x1, r1, 2, (n, n), (n, 1), (1, n))
    r2 = np.empty_like(x2)
    oracle.permute(x2, r2, 1, e2, ss2, ds2)
    assert np.array_equal(b1.cpu().numpy(), r1)
    assert np.array_equal(b2.cpu().numpy(), r2)
