#!/usr/bin/env python3
"""Benchmark of permute_layout on one MI355X.

Default workload: the batched scale-factor transpose, 2^20 independent 4x32
fp32 tiles (source strides (32, 1), destination (1, 4), tile stride 128
elements), 512 MiB in and 512 MiB out.  A step is one call of tpl_permute on
the whole batch, with the inputs already resident in HBM.  Source/destination
pairs rotate so that no step finds its data in the 256 MB Infinity Cache.

Prints ONE JSON line: whole-job GB/s (bytes read + written per second), the
roofline block of the dominant kernel (HIP-event time per launch on the
launch stream), the oracle's CPU throughput on the host, and the measured HBM
traffic from the committed rocprofv3 counter summary when it matches the
current kernel source.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --all]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "permute_layout GB/s (rd+wr) & % of HBM peak, batched 4x32 fp32 SF transpose"
PEAK_GBPS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 2 << 30      # src+dst bytes cycled through per rotation
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources of the profiled kernels and their planner (not the staged
# entry, which the counters do not cover).
_CSRC = os.path.join(ROOT, "tensor_layout_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.join(_CSRC, f) for f in os.listdir(_CSRC)
                        if f.endswith((".hip", ".hpp", ".cpp")) and f != "staged.hip")


def _code_only(text: str) -> str:
    """C/C++ source with comments and blank space removed, so that edits of
    comments alone keep the counters that were taken on the same code."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_for(name: str):
    """Counter-measured HBM bytes per launch, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_hash():
        return None
    rec = t.get("workloads", {}).get(name)
    if not rec:
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


def traffic_split_for(name: str):
    """The same counters split into HBM reads and writes, with their sum over
    the algorithmic bytes, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_hash():
        return None
    rec = t.get("workloads", {}).get(name)
    if not rec:
        return None
    return {"read_bytes": int(rec["fetch_bytes"]), "write_bytes": int(rec["write_bytes"]),
            "over_algorithmic": round((rec["fetch_bytes"] + rec["write_bytes"]) / rec["algorithmic_bytes"], 4)}


def lds_counters_for(name: str):
    """Per-dispatch LDS counters of the dominant kernel (rocprofv3), or None
    when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_hash():
        return None
    rec = t.get("lds", {}).get(name)
    if not rec:
        return None
    return rec


def dtype_name(w: int, specials: bool) -> str:
    return {1: "u8", 2: "u16", 4: "u32", 8: "u64", 16: "u128"}[w]


def buffer_bytes(wl):
    """(source, destination) buffer sizes in bytes: each side's element offset
    plus its batch of item spans (the cosize), widened to the reach of its
    swizzle.  Every byte a launch touches lies below these sizes."""
    from tensor_layout_amd import tpl

    def side(off, strides, z):
        if wl.elements == 0:
            return 0
        span = 1 + sum((e - 1) * st for e, st in zip(wl.extents, strides))
        return (off + tpl._swz_reach(wl.batch * span, z)) * wl.w

    return (side(wl.offsets[0], wl.src_strides, wl.src_swizzle),
            side(wl.offsets[1], wl.dst_strides, wl.dst_swizzle))


def make_input(wl):
    import numpy as np
    from tensor_layout_amd import synth
    x = synth.random_bytes(wl.seed, buffer_bytes(wl)[0]).copy()
    if wl.specials and wl.w == 4:
        synth.inject_f32_specials(x.view(np.uint32), wl.seed ^ 0x5EC1A1)
    return x


def host_info():
    """Host CPU model and the CPU count the process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def device_memory_props():
    """HBM clock and bus width as the HIP runtime reports them
    (hipDeviceGetAttribute, attributes hipDeviceAttributeMemoryClockRate = 60
    and hipDeviceAttributeMemoryBusWidth = 59 of hip_runtime_api.h), and the
    usual clock x width x 2 / 8 bandwidth formula on them.  On MI355X the
    runtime reports 2 GHz and 8192 bits: the formula, which assumes two
    transfers per pin per reported clock cycle, gives 4096 GB/s, half the
    published 8 TB/s (8192 pins at 8 Gb/s).  The published figure stays the
    peak."""
    import ctypes
    import torch
    try:
        lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        clk, bus = ctypes.c_int(), ctypes.c_int()
        if lib.hipDeviceGetAttribute(ctypes.byref(clk), 60, 0) or lib.hipDeviceGetAttribute(ctypes.byref(bus), 59, 0):
            return None
    except OSError:
        return None
    return {"memory_clock_khz": clk.value, "memory_bus_width_bits": bus.value,
            "clock_x_bus_x2_over_8_gbps": round(clk.value * 1e3 * bus.value * 2 / 8 / 1e9, 1)}


def device_info():
    """The device and software the line was measured on: the device name,
    its gfx target and CU count as torch reports them, the HIP runtime and
    driver versions (hipRuntimeGetVersion, hipDriverGetVersion) and torch's
    HIP build."""
    import ctypes
    import torch
    info = {}
    try:
        pr = torch.cuda.get_device_properties(0)
        info.update(name=pr.name, gcn_arch=getattr(pr, "gcnArchName", None),
                    compute_units=pr.multi_processor_count, total_memory_bytes=pr.total_memory)
    except Exception:   # noqa: BLE001 -- reported as absent
        pass
    try:
        lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        rt, drv = ctypes.c_int(), ctypes.c_int()
        if lib.hipRuntimeGetVersion(ctypes.byref(rt)) == 0:
            info["hip_runtime_version"] = rt.value
        if lib.hipDriverGetVersion(ctypes.byref(drv)) == 0:
            info["hip_driver_version"] = drv.value
    except OSError:
        pass
    info["torch_hip"] = getattr(torch.version, "hip", None)
    return info


def cpu_baseline(wl, x, min_seconds=10.0, max_runs=100):
    """The oracle as it stands, single-threaded, on the full workload."""
    import numpy as np
    import oracle
    y = np.zeros(buffer_bytes(wl)[1], dtype=np.uint8)
    # The calling thread is pinned to one of its cores while the oracle runs.
    pinned = None
    try:
        before = os.sched_getaffinity(0)
        pinned = min(before)
        os.sched_setaffinity(0, {pinned})
    except (AttributeError, OSError):
        before = None
    try:
        oracle.permute(x, y, wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
                       wl.src_swizzle, wl.dst_swizzle)   # untimed warm-up (first touch of the output)
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.permute(x, y, wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
                           wl.src_swizzle, wl.dst_swizzle)
            runs += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or runs >= max_runs:
                break
    finally:
        if before is not None:
            os.sched_setaffinity(0, before)
    return {
        "value": round(wl.bytes_moved * runs / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the full workload ({wl.elements} elements) permuted {runs} times by the "
                  f"single-threaded C oracle in {el:.1f} s",
        "host": dict(host_info(), pinned_core=pinned),
    }, y


def cpu_baseline_parallel(wl, x, y_ref, min_seconds=5.0, max_runs=200):
    """The same single-threaded C oracle run on all host cores at once, each
    thread on a slice of the workload (a range of batch items, or of the first
    mode when there is one item: the slice's element offsets move by the
    range start times the item span or the mode's strides, by the buffers
    page's address rule).  Plain layouts only (a swizzle acts on the
    unshifted layout offset).  Checked against the single-threaded result."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    if wl.src_swizzle or wl.dst_swizzle:
        return None
    threads = max(1, min(16, os.cpu_count() or 1))
    def cos(st):
        return 1 + sum((e - 1) * s_ for e, s_ in zip(wl.extents, st))
    if wl.batch > 1:
        n, unit_s, unit_d = wl.batch, cos(wl.src_strides), cos(wl.dst_strides)
    else:
        n, unit_s, unit_d = wl.extents[0], wl.src_strides[0], wl.dst_strides[0]
    cuts = [n * i // threads for i in range(threads + 1)]
    parts = [(a, b) for a, b in zip(cuts, cuts[1:]) if b > a]
    y = np.empty_like(y_ref)

    def one(ab):
        a, b = ab
        offs = (wl.offsets[0] + a * unit_s, wl.offsets[1] + a * unit_d)
        if wl.batch > 1:
            oracle.permute(x, y, wl.w, wl.extents, wl.src_strides, wl.dst_strides, offs, b - a)
        else:
            ext = (b - a,) + tuple(wl.extents[1:])
            oracle.permute(x, y, wl.w, ext, wl.src_strides, wl.dst_strides, offs, 1)

    with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        list(ex.map(one, parts))   # untimed: first touch of the output pages
        runs, t0 = 0, time.perf_counter()
        while True:
            list(ex.map(one, parts))
            runs += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or runs >= max_runs:
                break
    if not np.array_equal(y, y_ref):
        raise RuntimeError("parallel oracle run disagrees with the single-threaded one")
    return {
        "value": round(wl.bytes_moved * runs / el / 1e9, 4),
        "unit": "GB/s",
        "cores": len(parts),
        "kind": "oracle-parallel",
        "sample": f"the full workload permuted {runs} times in {el:.1f} s by {len(parts)} host threads, "
                  f"each running the single-threaded C oracle on a slice",
    }


def bench_one(wl, steps, warmup, do_cpu, do_verify, entry="permute", xor_k=-1, do_ceiling=True,
              cpu_seconds=(10.0, 5.0)):
    import numpy as np
    import torch
    from tensor_layout_amd import tpl

    dev = torch.device("cuda:0")
    x = make_input(wl)
    ns, nd = buffer_bytes(wl)
    if wl.inplace:
        # one buffer holds both layouts' footprints
        ns = nd = max(ns, nd)
        x = np.concatenate([x, np.zeros(ns - x.size, dtype=np.uint8)])
    nbytes = wl.elements * wl.w     # the bytes a launch moves each way
    pairs = max(2, min(128, math.ceil(ROTATE_BYTES / (ns + nd))))
    srcs = [torch.from_numpy(x).to(dev)]
    for _ in range(pairs - 1):
        srcs.append(srcs[0].clone())
    # In place: each step transposes its buffer again, so a buffer alternates
    # between the input and its transpose.
    dsts = srcs if wl.inplace else [torch.zeros(nd, dtype=torch.uint8, device=dev) for _ in range(pairs)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    plan = tpl.tpl_plan(wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
                        geometry=tpl.TPL_GEOM_GFX950_INPLACE if wl.inplace else tpl.TPL_GEOM_GFX950,
                        src_swizzle=wl.src_swizzle, dst_swizzle=wl.dst_swizzle)
    swz = (plan.k, plan.shift, plan.mask)
    if entry == "staged":
        # The staged entry runs the half-wave program on each batch item.
        hp = tpl.tpl_plan(wl.w, wl.extents, wl.src_strides, wl.dst_strides, (0, 0), 1,
                          geometry=tpl.TPL_GEOM_GFX950_HALFWAVE, src_swizzle=wl.src_swizzle,
                          dst_swizzle=wl.dst_swizzle)
        swz = (xor_k, 5 - xor_k, (1 << xor_k) - 1) if xor_k >= 0 else (hp.k, hp.shift, hp.mask)

    prepared = tpl.PreparedPermute(wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
                                   wl.src_swizzle, wl.dst_swizzle)
    ptrs = [(srcs[i].data_ptr(), dsts[i].data_ptr()) for i in range(pairs)]

    def launch(i):
        if entry == "staged":
            st = tpl.tpl_permute_staged(srcs[i % pairs].data_ptr(), dsts[i % pairs].data_ptr(), wl.w,
                                        wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
                                        xor_k, sp, wl.src_swizzle, wl.dst_swizzle)
        else:
            st = prepared(*ptrs[i % pairs], sp)
        if st != tpl.TPL_OK:
            raise tpl.TplError(st, tpl.tpl_last_error())

    # Reference first: a plain copy of the same bytes (the library's
    # identity-layout copy, 16-byte vectors) over the same buffer rotation,
    # 200 launches between two events after at least 30 ms of untimed ones.
    # Run before the warm-up, it also brings the GPU out of idle clocks, so
    # that a short timed run (a few launches) sees the same clocks as a long
    # one; the outputs it writes are cleared before the permute's launches.
    ceiling = None
    if do_ceiling and nbytes % 16 == 0 and nbytes <= min(ns, nd) and entry == "permute":
        ident = tpl.PreparedPermute(16, (nbytes // 16,), (1,), (1,))
        # in place, each source is copied onto the next (all hold the input)
        cptrs = [(srcs[i].data_ptr(), (srcs[(i + 1) % pairs] if wl.inplace else dsts[i]).data_ptr())
                 for i in range(pairs)]
        csteps = 200
        # untimed copies for at least 30 ms of GPU time, so that small
        # workloads are timed at load clocks too
        t_warm = time.perf_counter() + 0.03
        i = 0
        while i < 10 or time.perf_counter() < t_warm:
            for _ in range(10):
                ident(*cptrs[i % pairs], sp)
                i += 1
            torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for i in range(csteps):
            ident(*cptrs[i % pairs], sp)
        c1.record(stream)
        torch.cuda.synchronize()
        ceiling = 2 * nbytes / (c0.elapsed_time(c1) / csteps * 1e-3) / 1e9
        if not wl.inplace:
            for d in dsts:   # bytes outside the destination layout stay zero
                d.zero_()

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    # Two events on the launch stream bracket the K launches; the mean launch
    # duration is their interval / K (the host enqueues faster than the GPU
    # drains, so the queue stays full).  An event between every two launches
    # would add its own packet to each interval (about 1.5 us).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        launch(warmup + i)
    ev1.record(stream)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    avg_ms = ev0.elapsed_time(ev1) / steps
    host_us = (t_enq - t0) * 1e6 / steps
    elapsed = t1 - t0
    value = wl.bytes_moved * steps / elapsed / 1e9
    achieved = wl.bytes_moved / (avg_ms * 1e-3) / 1e9
    # A second, shorter pass with an event pair around every launch: the
    # spread of single launches (median, min, max).  Each interval also
    # holds one event packet, so these read a little above the mean above.
    nper = min(steps, 100)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nper)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        launch(warmup + steps + i)
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    per_launch = {"launches": nper, "median_ms": round(per[nper // 2], 5), "min_ms": round(per[0], 5),
                  "max_ms": round(per[-1], 5),
                  "median_gbps": round(wl.bytes_moved / (per[nper // 2] * 1e-3) / 1e9, 2)}


    out = {
        "metric": METRIC if wl.name == "sf_transpose_2^20x4x32_f32" else f"permute_layout GB/s (rd+wr), {wl.name}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed * 1e3 / steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name(wl.w, wl.specials),
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "elements": wl.elements,
            "element_bytes": wl.w,
            "bytes_per_step": wl.bytes_moved,
            "kernel": plan.kernel if entry == "permute" else "staged",
            "entry": "tpl_permute" if entry == "permute" else f"tpl_permute_staged(xor_k={xor_k})",
            "tile": list(plan.tile) if entry == "permute" else list(wl.extents),
            "k": swz[0], "shift": swz[1], "mask": swz[2],
            "buffer_pairs": pairs,
            **({"src_swizzle": list(wl.src_swizzle)} if wl.src_swizzle else {}),
            **({"dst_swizzle": list(wl.dst_swizzle)} if wl.dst_swizzle else {}),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": traffic_for(wl.name),
            "traffic_split": traffic_split_for(wl.name),
            "lds_counters": lds_counters_for(wl.name),
            "kernel_ms_avg": round(avg_ms, 5),
            "host_enqueue_us": round(host_us, 2),
            "per_launch": per_launch,
            "device_memory": device_memory_props(),
        },
        "device": device_info(),
    }
    ref = None
    if do_cpu:
        out["cpu_baseline"], ref = cpu_baseline(wl, x, min_seconds=cpu_seconds[0])
        out["cpu_baseline_parallel"] = cpu_baseline_parallel(wl, x, ref, min_seconds=cpu_seconds[1])
    if do_verify:
        import oracle
        if ref is None:
            ref = x.copy() if wl.inplace else np.zeros(nd, dtype=np.uint8)
            oracle.permute(x, ref, wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
                           wl.src_swizzle, wl.dst_swizzle)
        if wl.inplace:
            # one more call on a fresh copy of the input
            buf = torch.from_numpy(x).to(dev)
            st = prepared(buf.data_ptr(), buf.data_ptr(), sp)
            if st != tpl.TPL_OK:
                raise tpl.TplError(st, tpl.tpl_last_error())
            out["bitexact"] = bool(np.array_equal(buf.cpu().numpy(), ref))
        else:
            # the last output of every buffer pair that a launch wrote (all
            # pairs hold the same input, so all expect the oracle's output)
            written = min(pairs, warmup + steps + nper)
            out["bitexact"] = all(bool(np.array_equal(dsts[i].cpu().numpy(), ref)) for i in range(written))
            out["bitexact_pairs_checked"] = written
    # Warm: the same launches on one buffer pair, which then stays in the
    # 256 MB Infinity Cache when it fits (cache-assisted, not the HBM figure).
    if entry == "permute" and 2 * nbytes <= (200 << 20):
        p0 = ptrs[0]
        wsteps = min(steps, 200)
        for _ in range(10):
            prepared(*p0, sp)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(wsteps):
            prepared(*p0, sp)
        ev1.record(stream)
        torch.cuda.synchronize()
        out["warm_cache_assisted_gbps"] = round(wl.bytes_moved / (ev0.elapsed_time(ev1) / wsteps * 1e-3) / 1e9, 2)
    out["roofline"]["copy_ceiling_gbps"] = round(ceiling, 2) if ceiling else None
    out["roofline"]["frac_of_copy_ceiling"] = round(achieved / ceiling, 4) if ceiling else None
    del srcs, dsts
    torch.cuda.empty_cache()
    return out


def launches_only(wl, k, entry="permute", xor_k=-1):
    """K launches of one workload on uninitialised buffers, nothing timed or
    checked: the run a rocprofv3 counter pass wraps (counters serialise the
    kernels, and each workload's dispatches come out in this order)."""
    import torch
    from tensor_layout_amd import tpl
    dev = torch.device("cuda:0")
    ns, nd = buffer_bytes(wl)
    if wl.inplace:
        ns = nd = max(ns, nd)
    # Fresh buffer pairs in turn, as many as the benchmark's rotation uses
    # (up to K), so that small workloads stay out of the Infinity Cache too.
    pairs = max(1, min(k, max(2, min(128, math.ceil(ROTATE_BYTES / (ns + nd))))))
    srcs = [torch.empty(ns, dtype=torch.uint8, device=dev) for _ in range(pairs)]
    dsts = srcs if wl.inplace else [torch.empty(nd, dtype=torch.uint8, device=dev) for _ in range(pairs)]
    sp = torch.cuda.current_stream(dev).cuda_stream
    prepared = tpl.PreparedPermute(wl.w, wl.extents, wl.src_strides, wl.dst_strides, wl.offsets, wl.batch,
                                   wl.src_swizzle, wl.dst_swizzle)
    for i in range(k):
        src, dst = srcs[i % pairs], dsts[i % pairs]
        if entry == "staged":
            st = tpl.tpl_permute_staged(src.data_ptr(), dst.data_ptr(), wl.w, wl.extents, wl.src_strides,
                                        wl.dst_strides, wl.offsets, wl.batch, xor_k, sp, wl.src_swizzle,
                                        wl.dst_swizzle)
        else:
            st = prepared(src.data_ptr(), dst.data_ptr(), sp)
        if st != tpl.TPL_OK:
            raise tpl.TplError(st, tpl.tpl_last_error())
    torch.cuda.synchronize()
    print(f"launched {wl.name} x{k}", flush=True)
    del srcs, dsts
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="sf_transpose_2^20x4x32_f32")
    ap.add_argument("--all", action="store_true", help="one JSON line per workload")
    ap.add_argument("--rounds", type=int, default=1,
                    help="with --all: run the workloads interleaved this many rounds, drop the first "
                         "round (when more than one) and report each workload's median round")
    ap.add_argument("--with-calibration", action="store_true",
                    help="with --all: also run identity copies of 8, 16, 32, 64 and 512 MiB (the 512 MiB "
                         "one scales the HBM byte counters; all are same-size references)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the plain-copy reference (keeps profiler traces to the permute kernels)")
    ap.add_argument("--entry", choices=("permute", "staged"), default="permute",
                    help="tpl_permute (default) or the half-wave LDS-staged tpl_permute_staged")
    ap.add_argument("--xor-k", type=int, default=-1, help="staged entry: force this XOR k (-1 = planner's)")
    ap.add_argument("--launches-only", type=int, default=0, metavar="K",
                    help="K launches of the workload (or of every workload with --all, in list order) and "
                         "nothing else: the program a rocprofv3 counter pass wraps")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    from tensor_layout_amd import tpl, workloads
    tpl.load()
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    by_name = {w.name: w for w in workloads.ALL + workloads.INPLACE + workloads.COPY_REFERENCES}
    if a.launches_only:
        todo = (workloads.ALL + workloads.INPLACE + (workloads.COPY_REFERENCES if a.with_calibration else [])
                if a.all else [by_name[a.workload]])
        for wl in todo:
            launches_only(wl, a.launches_only, a.entry, a.xor_k)
        return
    if a.all:
        todo = workloads.ALL + workloads.INPLACE + (workloads.COPY_REFERENCES if a.with_calibration else [])
        # Every line carries the oracle's CPU throughput, on a shorter sample
        # than the single-workload run (about 3 s single-threaded, 2 s on all
        # host threads) so that the whole list stays within minutes.
        cpu_s = (3.0, 2.0)
        if a.rounds <= 1:
            for wl in todo:
                print(json.dumps(bench_one(wl, a.steps, a.warmup, not a.no_cpu, not a.no_verify,
                                           do_ceiling=not a.no_ceiling, cpu_seconds=cpu_s)), flush=True)
            return
        # Rounds over all workloads in turn; the first round only warms the
        # machine up.  Outputs are checked in the last round.
        kept = {wl.name: [] for wl in todo}
        for r in range(a.rounds):
            last = r == a.rounds - 1
            for wl in todo:
                out = bench_one(wl, a.steps, a.warmup, last and not a.no_cpu, last and not a.no_verify,
                                do_ceiling=last and not a.no_ceiling, cpu_seconds=cpu_s)
                print(f"round {r + 1}/{a.rounds} {wl.name}: {out['roofline']['achieved']} GB/s",
                      file=sys.stderr, flush=True)
                if r > 0:
                    kept[wl.name].append(out)
        for wl in todo:
            outs = sorted(kept[wl.name], key=lambda o: o["roofline"]["achieved"])
            med = dict(outs[len(outs) // 2])
            final = kept[wl.name][-1]
            for key in ("bitexact", "cpu_baseline", "cpu_baseline_parallel"):
                if key in final:
                    med[key] = final[key]
            roof = dict(med["roofline"])
            if final["roofline"].get("copy_ceiling_gbps"):
                roof["copy_ceiling_gbps"] = final["roofline"]["copy_ceiling_gbps"]
                roof["frac_of_copy_ceiling"] = round(roof["achieved"] / roof["copy_ceiling_gbps"], 4)
            roof["rounds"] = {"kept": len(outs), "dropped": 1,
                              "achieved_gbps": [o["roofline"]["achieved"] for o in kept[wl.name]]}
            med["roofline"] = roof
            print(json.dumps(med), flush=True)
        return
    wl = by_name[a.workload]
    print(json.dumps(bench_one(wl, a.steps, a.warmup, not a.no_cpu, not a.no_verify, a.entry, a.xor_k,
                               not a.no_ceiling)), flush=True)


if __name__ == "__main__":
    main()
