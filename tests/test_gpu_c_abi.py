"""The C ABI from a plain C++ program (tests/c_abi/abi_client.cpp, built by
build()): hipMalloc'd buffers, its own HIP stream, no Python or torch in the
process that calls the library.  Its output is compared with the oracle."""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from tensor_layout_amd import synth, tpl

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_client")


def _cos(ext, st):
    return 1 + sum((e - 1) * s for e, s in zip(ext, st))


def run_client(tmp_path, name, w, ext, ss, ds, offs=(0, 0), batch=1, zs=None, zd=None, staged_k=None):
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_abi/abi_client is missing: run build() first")
    print(f"\n[case] C client {name}: w={w} ext={ext} ss={ss} ds={ds} offs={offs} batch={batch} "
          f"zs={zs} zd={zd} staged_k={staged_k}", flush=True)
    ns = (offs[0] + batch * _cos(ext, ss)) * w
    nd = (offs[1] + batch * _cos(ext, ds)) * w
    x = synth.random_bytes(len(name), ns).copy()
    ref = np.full(nd, 0xA5, dtype=np.uint8)
    oracle.permute(x, ref, w, ext, ss, ds, offs, batch, zs, zd)
    fin, fout = tmp_path / f"{name}.in", tmp_path / f"{name}.out"
    x.tofile(fin)
    args = [CLIENT, str(fin), str(fout), str(w), str(len(ext))] + [str(v) for v in (*ext, *ss, *ds)] + \
        [str(offs[0]), str(offs[1]), str(batch), str(nd)]
    if zs is not None or zd is not None:
        z0, z1 = zs or (0, 0, 0), zd or (0, 0, 0)
        args.append("swz:%d,%d,%d:%d,%d,%d" % (*z0, *z1))
    elif staged_k is not None:
        args.append(f"staged:{staged_k}")
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    print(r.stdout.strip(), r.stderr.strip(), flush=True)
    return r, fout, ref


@pytest.mark.parametrize("case", [
    ("sf_fp32", 4, (4, 32), (32, 1), (1, 4), (0, 0), 4096),
    ("tiles_fp16", 2, (128, 64), (64, 1), (1, 128), (0, 0), 8),
    ("bf16_1000x700_offsets", 2, (1000, 700), (700, 1), (1, 1000), (8, 24), 1),
    ("u8_axes0231", 1, (4, 128, 32, 32), (131072, 1024, 32, 1), (131072, 1, 4096, 128), (0, 0), 1),
    ("u128_300x200", 16, (300, 200), (200, 1), (1, 300), (0, 0), 1),
    ("rec_float3_aos_to_soa", 4, (3000, 3), (3, 1), (1, 3000), (0, 0), 1),
    ("etile_bf16_odd_pitch", 2, (300, 500), (501, 1), (1, 300), (0, 0), 1),
    ("copy_row_blocks_f32", 4, (8, 16, 256), (4096, 256, 1), (256, 2048, 1), (0, 0), 1),
    ("quad_u8_sf", 1, (4, 32), (32, 1), (1, 4), (0, 0), 2048),
    ("gather_no_unit_stride", 4, (16, 24), (48, 2), (24, 1), (0, 0), 1),
], ids=lambda c: c[0])
def test_c_client_matches_oracle(tmp_path, case):
    name, w, ext, ss, ds, offs, batch = case
    r, fout, ref = run_client(tmp_path, name, w, ext, ss, ds, offs, batch)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
    got = np.fromfile(fout, dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_c_client_decline(tmp_path):
    # destination with repeated addresses: declined before any launch
    sp = tmp_path
    name, w, ext, ss, ds = "decline", 4, (4, 32), (32, 1), (1, 2)
    x = synth.random_bytes(1, 128 * 4).copy()
    (sp / "decline.in").write_bytes(x.tobytes())
    args = [CLIENT, str(sp / "decline.in"), str(sp / "decline.out"), "4", "2", "4", "32", "32", "1", "1", "2",
            "0", "0", "1", "512"]
    print("\n[case] C client decline", flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=60)
    assert r.returncode == 4 and f"status={tpl.TPL_E_LAYOUT}" in r.stdout, r.stdout


@pytest.mark.parametrize("case", [
    # (name, w, extents, src strides, dst strides, batch, src swizzle, dst swizzle)
    ("sf_fp32_into_swizzled", 4, (4, 32), (32, 1), (1, 4), 512, None, (2, 2, 3)),
    ("tiles_fp16_from_swizzled", 2, (128, 64), (64, 1), (1, 128), 4, (3, 3, 4), None),
    ("bf16_element_form_swizzled", 2, (256, 256), (256, 1), (1, 256), 1, (3, 2, 3), None),
], ids=lambda c: c[0])
def test_c_client_swizzled_matches_oracle(tmp_path, case):
    """tpl_plan_swizzled and tpl_permute_swizzled from the plain C++ client."""
    name, w, ext, ss, ds, batch, zs, zd = case
    r, fout, ref = run_client(tmp_path, name, w, ext, ss, ds, (0, 0), batch, zs=zs, zd=zd)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
    assert np.array_equal(np.fromfile(fout, dtype=np.uint8), ref)


@pytest.mark.parametrize("case", [
    # (name, w, extents, src strides, dst strides, batch, xor_k)
    ("staged_sf_fp32", 4, (4, 32), (32, 1), (1, 4), 7001, -1),
    ("staged_sf_fp32_k0", 4, (4, 32), (32, 1), (1, 4), 301, 0),
    ("staged_8x32_fp16", 2, (8, 32), (32, 1), (1, 8), 1001, -1),
], ids=lambda c: c[0])
def test_c_client_staged_matches_oracle(tmp_path, case):
    """tpl_permute_staged (the pages' half-wave program) from the plain C++
    client, with the planner's k and with the swizzle forced off."""
    name, w, ext, ss, ds, batch, k = case
    r, fout, ref = run_client(tmp_path, name, w, ext, ss, ds, (0, 0), batch, staged_k=k)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
    assert np.array_equal(np.fromfile(fout, dtype=np.uint8), ref)
