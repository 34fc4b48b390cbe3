"""HIP graph capture of every kernel family at sizes that take the launch-size
dependent choices (occupancy reserves, the pipelined staged loop): each call
is captured once into one graph, which is replayed three times on new inputs
with eager work and host synchronisations in between; every replay's output
equals the oracle's, byte for byte."""

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


def _cos(ext, st):
    return 1 + sum((e - 1) * s for e, s in zip(ext, st))


# (name, w, extents, src strides, dst strides, batch, src swizzle, expected kernel)
OUT_OF_PLACE = [
    ("lds_bf16_4096sq_strided", 2, (4096, 4096), (4096, 1), (1, 4096), 1, None, "lds"),
    ("etile_bf16_8192sq_pitch8196", 2, (8192, 8192), (8196, 1), (1, 8192), 1, None, "etile"),
    ("etile_swizzled_bf16_1024sq", 2, (1024, 1024), (1024, 1), (1, 1024), 1, (3, 2, 3), "etile"),
    ("etile_tall_bf16_8192sq_dst_pitch8193", 2, (8192, 8192), (8192, 1), (1, 8193), 1, None, "etile"),
    ("rec_float3_2p20", 4, (1 << 20, 3), (3, 1), (1, 1 << 20), 1, None, "rec"),
    ("copy_runs_f32", 4, (64, 128, 1024), (131072, 1024, 1), (1024, 65536, 1), 1, None, "copy"),
    ("quad_u8_sf", 1, (4, 32), (32, 1), (1, 4), 1 << 16, None, "quad"),
]


def test_graph_replays_every_kernel_family():
    torch = _torch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    cases = []
    for name, w, ext, ss, ds, batch, zs, kernel in OUT_OF_PLACE:
        p = tpl.tpl_plan(w, ext, ss, ds, (0, 0), batch, src_swizzle=zs)
        assert p.ok and p.kernel == kernel, (name, p)
        ns, nd = batch * _cos(ext, ss) * w, batch * _cos(ext, ds) * w
        src = torch.zeros(ns, dtype=torch.uint8, device="cuda")
        dst = torch.zeros(nd, dtype=torch.uint8, device="cuda")
        cases.append((name, w, ext, ss, ds, batch, zs, src, dst))
    # in place: 8192^2 bf16 (8256 tile pairs: the pair-swap occupancy reserve)
    n = 8192
    ip = torch.zeros(n * n * 2, dtype=torch.uint8, device="cuda")
    p = tpl.tpl_plan(2, (n, n), (n, 1), (1, n), geometry=tpl.TPL_GEOM_GFX950_INPLACE)
    assert p.ok and p.kernel == "swap", p
    # staged: 3 x 6144 + 1001 SF tiles (the pipelined loop and a tail)
    sb = 3 * 6144 + 1001
    s_src = torch.zeros(sb * 512, dtype=torch.uint8, device="cuda")
    s_dst = torch.zeros(sb * 512, dtype=torch.uint8, device="cuda")

    def calls():
        for name, w, ext, ss, ds, batch, zs, src, dst in cases:
            tpl.permute(dst, src, ext, ss, ds, batch=batch, dtype_bytes=w, src_swizzle=zs)
        tpl.permute(ip, ip, (n, n), (n, 1), (1, n), dtype_bytes=2)
        st = tpl.tpl_permute_staged(s_src.data_ptr(), s_dst.data_ptr(), 4, (4, 32), (32, 1), (1, 4), (0, 0), sb,
                                    -1, side.cuda_stream)
        assert st == tpl.TPL_OK, tpl.tpl_last_error()

    print("\n[case] graph: " + ", ".join(c[0] for c in OUT_OF_PLACE) + ", swap 8192^2, staged", flush=True)
    with torch.cuda.stream(side):
        calls()   # plans are made outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls()
    for rep in range(3):
        inputs = []
        for k, (name, w, ext, ss, ds, batch, zs, src, dst) in enumerate(cases):
            x = synth.random_bytes(1000 * rep + k, src.numel()).copy()
            src.copy_(torch.from_numpy(x))
            dst.fill_(0)
            inputs.append(x)
        xi = synth.random_bytes(1000 * rep + 77, ip.numel()).copy()
        ip.copy_(torch.from_numpy(xi))
        xs = synth.random_bytes(1000 * rep + 88, s_src.numel()).copy()
        s_src.copy_(torch.from_numpy(xs))
        s_dst.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, w, ext, ss, ds, batch, zs, src, dst), x in zip(cases, inputs):
            ref = np.zeros(dst.numel(), dtype=np.uint8)
            oracle.permute(x, ref, w, ext, ss, ds, (0, 0), batch, zs, None)
            assert np.array_equal(dst.cpu().numpy(), ref), (name, rep)
        ref = xi.copy()
        oracle.permute(xi, ref, 2, (n, n), (n, 1), (1, n), (0, 0), 1)
        assert np.array_equal(ip.cpu().numpy(), ref), ("swap", rep)
        ref = np.zeros(s_dst.numel(), dtype=np.uint8)
        oracle.permute(xs, ref, 4, (4, 32), (32, 1), (1, 4), (0, 0), sb)
        assert np.array_equal(s_dst.cpu().numpy(), ref), ("staged", rep)
