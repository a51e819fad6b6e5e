"""Throughput of in-place partial RoPE on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c4|c3|c4_f32|...]

One step = one backward and one forward launch over the whole workload (the
full hot path: argument checks, index mapping, loads, fp32 rotation,
round-to-nearest-even stores), in place, inputs resident in HBM. The default
workload is the long-context backward shard: dx (16,8192,32,128) bf16, slice
[32,96), interleave, per-batch position tables (16,8192,1,64) with base 5e5.

Prints one JSON line: whole-job algorithmic GB/s (slice read + slice written +
cos/sin read once, per launch) and Gelem/s, the roofline of the dominant
kernel (average launch duration from HIP events on the launch stream), HBM
traffic from the committed rocprofv3 counter summary when it matches the
current kernel source (and, per kernel, the measured HBM bytes per second
as a fraction of peak), and the CPU oracle timed on a bounded sample.

`--profile-target` runs only launches of the chosen kernel plus a copy of
known size (for rocprofv3 counter passes), and prints nothing else.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of MI355X peak) + Gelem/s, partial-RoPE fwd/bwd in place"
PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public spec
KERNEL_DIR = os.path.join(ROOT, "transformer_positional_encoding_amd", "csrc")
TRAFFIC_MD = os.path.join(ROOT, "profiles", "rope_kernels_hbm_traffic_by_workload.md")


def kernel_source_hash() -> str:
    """sha256[:16] of the library's sources (every file of csrc/, in name
    order) with comments and spacing removed: editing a comment keeps the
    committed counters valid, changing code makes them stale."""
    text = ""
    for name in sorted(os.listdir(KERNEL_DIR)):
        if name.endswith((".hip", ".hpp", ".cpp", ".h")):
            with open(os.path.join(KERNEL_DIR, name), encoding="utf-8") as f:
                text += f"\n// {name}\n" + f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def committed_traffic(workload: str, direction: str):
    """Per-launch HBM bytes (read, write) measured by rocprofv3 for this
    kernel source, from profiles/rope_kernels_hbm_traffic_by_workload.md; None if absent or stale."""
    if not os.path.exists(TRAFFIC_MD):
        return None
    text = open(TRAFFIC_MD, encoding="utf-8").read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    if data.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    entry = data.get("launches", {}).get(f"{workload}:{direction}")
    return entry


def launch_fn(direction):
    import transformer_positional_encoding_amd as rp
    return rp.rope_partial_fwd_inplace if direction == "fwd" else rp.rope_partial_bwd_inplace


def time_launches(calls, n: int, stream) -> float:
    """Average duration (s) of n back-to-back launches on `stream`, taking
    the (fn, args) pairs of `calls` in turn, from HIP events recorded on that
    same stream."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n):
        fn, args = calls[i % len(calls)]
        fn(*args)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / n


def settle(launch, min_launches: int = 200, min_seconds: float = 0.15) -> dict:
    """Keep the GPU busy with untimed launches (launch(j) issues launch j)
    until at least min_launches have run and min_seconds have passed. After
    any idle period (host-side data generation, even 50 ms of nothing) the
    first ~80 launches of an HBM-bound kernel on MI355X run 5-40% slow while
    the memory clocks ramp; timing them would measure the ramp."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < min_launches or time.perf_counter() - t0 < min_seconds:
        for _ in range(20):
            launch(n)
            n += 1
        torch.cuda.synchronize()
    return {"launches": n, "seconds": round(time.perf_counter() - t0, 3)}


MALL_BYTES = 256 << 20  # MI355X Infinity Cache


def slice_line_bytes(w, k: int = 0) -> int:
    """Bytes of the 128-byte lines that one launch's slice touches in x."""
    import workloads as W
    B, S, N, D = w.x_shapes[k]
    es = W.ESIZE[w.dtype]
    lo = (w.partial_slice[0] * es) // 128 * 128
    hi = -(-(w.partial_slice[1] * es) // 128) * 128
    return B * S * N * (hi - lo)


def rotating_copies(w) -> int:
    """How many copies of x the timed launches rotate over so that each
    launch reads lines the 256 MB MALL no longer holds (>= 3x its size)."""
    return max(1, min(8, -(-(3 * MALL_BYTES) // slice_line_bytes(w))))


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x_cpu, r1, r2, directions, budget_s: float, max_threads: int = 16) -> dict:
    """The CPU oracle as written, running the GPU's step (every direction of
    the workload, in order) on the same data. Timed single-threaded, then
    with the rows split into contiguous blocks over the host cores (one
    thread per block, each calling the oracle on its rows; the oracle
    releases the interpreter while it runs). Whole-tensor steps are repeated
    to fill ~budget_s per timing, or the first rows are taken when one step
    would take longer."""
    import threading

    import numpy as np

    import oracle
    import workloads as W

    B, S, N, D = (int(v) for v in x_cpu.shape)
    total = B * S * N
    flat = W.to_numpy_storage(x_cpu).reshape(-1, D)
    t1, t2 = W.to_numpy_storage(r1), W.to_numpy_storage(r2)
    per_row = 2 * w.L * W.ESIZE[w.dtype]

    def step(buf, rows):
        for d in directions:
            oracle.rope_rows(buf, x_cpu.shape, w.dtype, t1, t2, w.mode, w.partial_slice, d, rows=rows)

    def run(nrows, threads):
        bounds = np.linspace(0, nrows, threads + 1).astype(np.int64)
        parts = [(np.ascontiguousarray(flat[a:b]), np.arange(a, b, dtype=np.int64))
                 for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        workers = [threading.Thread(target=step, args=part) for part in parts]
        t0 = time.perf_counter()
        for th in workers:
            th.start()
        for th in workers:
            th.join()
        return time.perf_counter() - t0

    def timed(threads):
        n_cal = min(total, 20000 * threads)
        rate = n_cal / max(run(n_cal, threads), 1e-9)          # rows per second, one step
        if total / rate <= budget_s:
            nrows, reps = total, max(1, int(budget_s * rate / total))
        else:
            nrows, reps = max(n_cal, int(rate * budget_s)), 1
        dt = sum(run(nrows, threads) for _ in range(reps))
        groups = -(-nrows // N)
        table_bytes = 2 * groups * w.L * W.ESIZE[w.tdtype]
        moved = reps * len(directions) * (nrows * per_row + table_bytes)
        return moved / dt / 1e9, nrows, reps, dt

    cores = max(1, min(len(os.sched_getaffinity(0)), max_threads))
    one = timed(1)
    many = timed(cores) if cores > 1 else one
    gbps, nrows, reps, dt = many
    what = "all" if nrows == total else f"the first {nrows} of {total}"
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} step(s) of {'+'.join(directions)} over {what} rows of the workload, rows split "
                      f"over {cores} threads, {dt:.1f} s; bytes counted as on the GPU",
            "single_core_value": round(one[0], 4),
            "single_core_sample": f"{one[2]} step(s) over {'all' if one[1] == total else one[1]} rows, "
                                  f"{one[3]:.1f} s on one thread",
            "cpu_model": host_cpu_model(), "host_cores_available": len(os.sched_getaffinity(0))}


def bench_workload(name: str, steps: int, warmup: int, reps: int, stream, want_cpu: bool, cpu_s: float):
    import torch

    import workloads as W
    w = W.WORKLOADS[name]
    x_cpu = W.make_x(w)
    r1, r2 = W.make_tables(w)
    ncopy = rotating_copies(w)
    xs = [x_cpu.to("cuda")]
    xs += [xs[0].clone() for _ in range(ncopy - 1)]
    r1d, r2d = r1.to("cuda"), r2.to("cuda")
    torch.cuda.synchronize()
    # a step runs both directions, the workload's own direction first
    dirs = list(w.directions) + [d for d in ("fwd", "bwd") if d not in w.directions]
    step_calls = [(launch_fn(d), (None, r1d, r2d, w.mode, w.partial_slice)) for d in dirs]

    def launches(i0, n):
        # launch j works on copy j % ncopy: no launch finds its data in a cache
        for j in range(i0, i0 + n):
            fn, args = step_calls[j % len(dirs)]
            fn(xs[j % ncopy], *args[1:])

    settled = settle(lambda j: launches(j, 1))
    launches(0, warmup * len(dirs))
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    launches(0, steps * len(dirs))
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_s = ev0.elapsed_time(ev1) / 1e3 / steps
    # per-kernel average launch durations: rotating copies (data from HBM),
    # and back to back on one buffer (what caches keep of it is reused)
    # Two rounds over the directions, the second kept: the first launches
    # after a workload's data is generated read a few percent slow, and the
    # first direction timed would otherwise take all of that.
    per_launch, warm = {}, {}
    for _ in range(2):
        for d in dirs:
            fn = launch_fn(d)
            cold = [(fn, (xs[i], r1d, r2d, w.mode, w.partial_slice)) for i in range(ncopy)]
            time_launches(cold, max(10, reps // 2), stream)  # untimed: settle clocks after the host gap
            per_launch[d] = time_launches(cold, reps, stream)
            warm[d] = time_launches(cold[:1], reps, stream)
    bytes_launch = w.algorithmic_bytes()
    elems_launch = w.rotated_elements()
    out = {
        "workload": name, "note": w.note, "x_shape": list(w.x_shapes[0]), "dtype": w.dtype,
        "slice": list(w.partial_slice), "mode": w.mode, "table_shape": list(w.table_shape),
        "directions": dirs, "step_s": step_s, "wall_s": wall, "rotating_copies": ncopy, "settle": settled,
        "bytes_per_launch": bytes_launch, "elements_per_launch": elems_launch,
        "kernels": {d: {"avg_launch_us": round(t * 1e6, 3),
                        "GBps": round(bytes_launch / t / 1e9, 1),
                        "Gelem_per_s": round(elems_launch / t / 1e9, 1),
                        "frac_of_peak": round(bytes_launch / t / 1e9 / PEAK_GBPS, 4),
                        "same_buffer_avg_launch_us": round(warm[d] * 1e6, 3)}
                    for d, t in per_launch.items()},
    }
    # The same launches in measured HBM bytes (rocprofv3 counters of this
    # kernel source), when they are committed.
    for d, t in per_launch.items():
        tr = committed_traffic(name, d)
        if tr is not None:
            k = out["kernels"][d]
            k["hbm_bytes_per_launch"] = tr["hbm_bytes_per_launch"]
            k["hbm_GBps"] = round(tr["hbm_bytes_per_launch"] / t / 1e9, 1)
            k["hbm_frac_of_peak"] = round(tr["hbm_bytes_per_launch"] / t / 1e9 / PEAK_GBPS, 4)
    if want_cpu:
        out["cpu_baseline"] = cpu_baseline(w, x_cpu, r1, r2, dirs, cpu_s)
    del xs, x_cpu
    torch.cuda.empty_cache()
    return out


def bench_multi(name: str, reps: int, stream) -> dict:
    """A workload with several tensors (the GQA Q and K): forward launch time
    of one _multi call against one single-tensor call per tensor, rotating
    copies so that no launch finds its data in a cache."""
    import torch

    import transformer_positional_encoding_amd as rp
    import workloads as W
    w = W.WORKLOADS[name]
    r1, r2 = (t.to("cuda") for t in W.make_tables(w))
    per_set = sum(slice_line_bytes(dataclasses.replace(w, x_shapes=(shp,))) for shp in w.x_shapes)
    ncopy = max(1, min(8, -(-(3 * MALL_BYTES) // per_set)))
    base = [W.make_x(w, k).to("cuda") for k in range(len(w.x_shapes))]
    sets = [[t.clone() for t in base] for _ in range(ncopy)]
    one = [(rp.rope_partial_fwd_inplace_multi, (sets[i], r1, r2, w.mode, w.partial_slice)) for i in range(ncopy)]
    each = [(lambda xs: [rp.rope_partial_fwd_inplace(x, r1, r2, w.mode, w.partial_slice) for x in xs], (sets[i],))
            for i in range(ncopy)]
    time_launches(one, max(4, reps // 4), stream)
    t_one = time_launches(one, reps, stream)
    time_launches(each, max(4, reps // 4), stream)
    t_each = time_launches(each, reps, stream)
    nbytes = w.algorithmic_bytes()
    return {"workload": name, "note": w.note, "dtype": w.dtype, "directions": ["fwd"], "rotating_copies": ncopy,
            "bytes_per_call": nbytes, "elements_per_call": w.rotated_elements(),
            "one_launch_us": round(t_one * 1e6, 3), "one_launch_GBps": round(nbytes / t_one / 1e9, 1),
            "separate_launches_us": round(t_each * 1e6, 3),
            "separate_launches_GBps": round(nbytes / t_each / 1e9, 1)}


def bench_pos_multi(name: str, reps: int, stream) -> dict:
    """A workload with several tensors (the GQA Q and K) through the
    position entry points: forward launch time of one _pos_multi call (cos
    and sin evaluated once per position for both tensors) against one
    position call per tensor, rotating copies as bench_multi does."""
    import torch

    import transformer_positional_encoding_amd as rp
    import workloads as W
    w = W.WORKLOADS[name]
    pos = torch.from_numpy(W.positions(w)).to("cuda")
    f = rp.rope_inv_freq(w.L, w.base, "cuda")
    per_set = sum(slice_line_bytes(dataclasses.replace(w, x_shapes=(shp,))) for shp in w.x_shapes)
    ncopy = max(1, min(8, -(-(3 * MALL_BYTES) // per_set)))
    base = [W.make_x(w, k).to("cuda") for k in range(len(w.x_shapes))]
    sets = [[t.clone() for t in base] for _ in range(ncopy)]
    one = [(rp.rope_partial_fwd_inplace_pos_multi, (sets[i], pos, f, w.mode, w.partial_slice)) for i in range(ncopy)]
    each = [(lambda xs: [rp.rope_partial_fwd_inplace_pos(x, pos, f, w.mode, w.partial_slice) for x in xs], (sets[i],))
            for i in range(ncopy)]
    time_launches(one, max(4, reps // 4), stream)
    t_one = time_launches(one, reps, stream)
    time_launches(each, max(4, reps // 4), stream)
    t_each = time_launches(each, reps, stream)
    nbytes = sum(2 * B * S * N * w.L * W.ESIZE[w.dtype] for (B, S, N, _) in w.x_shapes) + pos.numel() * 8 + f.numel() * 8
    return {"workload": name, "note": w.note + ", tables computed from positions", "dtype": w.dtype,
            "directions": ["fwd"], "rotating_copies": ncopy, "bytes_per_call": nbytes,
            "elements_per_call": w.rotated_elements(),
            "one_launch_us": round(t_one * 1e6, 3), "one_launch_GBps": round(nbytes / t_one / 1e9, 1),
            "separate_launches_us": round(t_each * 1e6, 3),
            "separate_launches_GBps": round(nbytes / t_each / 1e9, 1)}


def bench_out_of_place(name: str, reps: int, stream) -> dict:
    """The out-of-place entry points on a workload (what the autograd ops
    run: the backward writes the gradient with respect to x into a new
    buffer and leaves the incoming gradient alone). Launch time of one
    out-of-place call against the two-step alternative it replaces, a
    device copy of x followed by the in-place call. Bytes per call: x read
    whole, the result written whole, the tables read once."""
    import torch

    import transformer_positional_encoding_amd as rp
    import workloads as W
    w = W.WORKLOADS[name]
    x = W.make_x(w).to("cuda")
    r1, r2 = (t.to("cuda") for t in W.make_tables(w))
    B, S, N, D = w.x_shapes[0]
    es = W.ESIZE[w.dtype]
    whole = B * S * N * D * es
    ncopy = max(1, min(4, -(-(3 * MALL_BYTES) // whole)))
    xs = [x] + [x.clone() for _ in range(ncopy - 1)]
    ys = [torch.empty_like(x) for _ in range(ncopy)]
    nbytes = 2 * whole + (w.algorithmic_bytes() - 2 * B * S * N * w.L * es)
    res = {"workload": name, "note": w.note + ", out of place", "dtype": w.dtype, "rotating_copies": ncopy,
           "bytes_per_call": nbytes, "kernels": {}}
    for d in ("bwd", "fwd"):
        out_fn = rp.rope_partial_bwd_out if d == "bwd" else rp.rope_partial_fwd_out
        in_fn = launch_fn(d)
        one = [(out_fn, (ys[i], xs[i], r1, r2, w.mode, w.partial_slice)) for i in range(ncopy)]

        def copy_then_in_place(y, src):
            y.copy_(src)
            in_fn(y, r1, r2, w.mode, w.partial_slice)

        two = [(copy_then_in_place, (ys[i], xs[i])) for i in range(ncopy)]
        time_launches(one, max(4, reps // 4), stream)
        t_one = time_launches(one, reps, stream)
        time_launches(two, max(4, reps // 4), stream)
        t_two = time_launches(two, reps, stream)
        res["kernels"][d] = {"out_of_place_us": round(t_one * 1e6, 3),
                             "GBps": round(nbytes / t_one / 1e9, 1),
                             "frac_of_peak": round(nbytes / t_one / 1e9 / PEAK_GBPS, 4),
                             "copy_then_in_place_us": round(t_two * 1e6, 3)}
        tr = committed_traffic(name + ":out", d)
        if tr is not None:
            res["kernels"][d]["hbm_bytes_per_launch"] = tr["hbm_bytes_per_launch"]
            res["kernels"][d]["hbm_GBps"] = round(tr["hbm_bytes_per_launch"] / t_one / 1e9, 1)
            res["kernels"][d]["hbm_frac_of_peak"] = round(tr["hbm_bytes_per_launch"] / t_one / 1e9 / PEAK_GBPS, 4)
    del xs, ys, x
    torch.cuda.empty_cache()
    return res


def bench_positions(name: str, reps: int, stream, out: bool = False) -> dict:
    """The position entry points on a workload: cos and sin computed in the
    kernel from the workload's positions (one int64 per (b,s)) and its L/2
    double frequencies, against the table call on the same x. Bytes per
    launch: the slice read and written once (out of place: x read whole and
    the result written whole), the positions and frequencies read once (no
    tables). Rotating copies as for the table call."""
    import torch

    import transformer_positional_encoding_amd as rp
    import workloads as W
    w = W.WORKLOADS[name]
    B, S, N, D = w.x_shapes[0]
    es = W.ESIZE[w.dtype]
    whole = B * S * N * D * es
    ncopy = max(1, min(4, -(-(3 * MALL_BYTES) // whole))) if out else rotating_copies(w)
    xs = [W.make_x(w).to("cuda")]
    xs += [xs[0].clone() for _ in range(ncopy - 1)]
    ys = [torch.empty_like(xs[0]) for _ in range(ncopy)] if out else xs
    pos = torch.from_numpy(W.positions(w)).to("cuda")
    f = rp.rope_inv_freq(w.L, w.base, "cuda")
    r1, r2 = (t.to("cuda") for t in W.make_tables(w))
    moved = 2 * whole if out else 2 * B * S * N * w.L * es
    nbytes = moved + pos.numel() * 8 + f.numel() * 8
    table_bytes = moved + (w.algorithmic_bytes() - 2 * B * S * N * w.L * es)
    tdt = W.TORCH_DTYPES[w.tdtype]
    res = {"workload": name, "note": w.note + (", out of place" if out else "") + ", tables computed from positions",
           "dtype": w.dtype, "table_dtype": w.tdtype, "rotating_copies": ncopy, "bytes_per_launch": nbytes,
           "table_call_bytes_per_launch": table_bytes, "kernels": {}}
    for _ in range(2):   # two rounds, the second kept (as for the table call)
        for d in ("bwd", "fwd"):
            if out:
                pos_fn = rp.rope_partial_bwd_out_pos if d == "bwd" else rp.rope_partial_fwd_out_pos
                tab_fn = rp.rope_partial_bwd_out if d == "bwd" else rp.rope_partial_fwd_out
                with_pos = [(pos_fn, (ys[i], xs[i], pos, f, w.mode, w.partial_slice, tdt)) for i in range(ncopy)]
                with_tables = [(tab_fn, (ys[i], xs[i], r1, r2, w.mode, w.partial_slice)) for i in range(ncopy)]
            else:
                pos_fn = rp.rope_partial_bwd_inplace_pos if d == "bwd" else rp.rope_partial_fwd_inplace_pos
                with_pos = [(pos_fn, (xs[i], pos, f, w.mode, w.partial_slice, tdt)) for i in range(ncopy)]
                with_tables = [(launch_fn(d), (xs[i], r1, r2, w.mode, w.partial_slice)) for i in range(ncopy)]
            time_launches(with_pos, max(10, reps // 2), stream)
            t_pos = time_launches(with_pos, reps, stream)
            time_launches(with_tables, max(10, reps // 2), stream)
            t_tab = time_launches(with_tables, reps, stream)
            res["kernels"][d] = {"positions_us": round(t_pos * 1e6, 3), "GBps": round(nbytes / t_pos / 1e9, 1),
                                 "frac_of_peak": round(nbytes / t_pos / 1e9 / PEAK_GBPS, 4),
                                 "table_call_us": round(t_tab * 1e6, 3)}
            tr = committed_traffic(name + (":outpos" if out else ":pos"), d)
            if tr is not None:
                res["kernels"][d]["hbm_bytes_per_launch"] = tr["hbm_bytes_per_launch"]
                res["kernels"][d]["hbm_GBps"] = round(tr["hbm_bytes_per_launch"] / t_pos / 1e9, 1)
                res["kernels"][d]["hbm_frac_of_peak"] = round(
                    tr["hbm_bytes_per_launch"] / t_pos / 1e9 / PEAK_GBPS, 4)
    del xs, ys
    torch.cuda.empty_cache()
    return res


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA, AMD public spec


def bench_proj(name: str, reps: int, stream) -> dict:
    """The projection with a rotary epilogue (rope_proj_fwd) on a workload,
    against the ways to get the same result in two steps: this library's
    projection without the rotation (an empty slice) or torch's matmul
    (hipBLASLt), each followed by the in-place rotation of the result. The
    fused call also rotates the fp32 accumulator rather than a rounded
    result (the two-step results may differ by a unit in the last place)."""
    import torch

    import transformer_positional_encoding_amd as rp
    import workloads as W
    pw = W.PROJ_WORKLOADS[name]
    wr = W.WORKLOADS[pw.rope]
    B, S, H, Dh = pw.y_shape
    x, w = (t.to("cuda") for t in W.make_proj_inputs(pw))
    r1, r2 = (t.to("cuda") for t in W.make_tables(wr))
    z = torch.zeros((1, 1, 1, 0), dtype=x.dtype, device="cuda")
    y = torch.empty((B, S, H, Dh), dtype=x.dtype, device="cuda")
    y2 = y.view(B * S, H * Dh)
    x2, wt = x.view(B * S, pw.K), w.t()
    sl, mode = wr.partial_slice, wr.mode

    def fused():
        rp.rope_proj_fwd(x, w, r1, r2, H, mode, sl, out=y)

    def plain():
        rp.rope_proj_fwd(x, w, z, z, H, mode, None, out=y)

    def plain_then_rope():
        plain()
        rp.rope_partial_fwd_inplace(y, r1, r2, mode, sl)

    def torch_mm():
        torch.matmul(x2, wt, out=y2)

    def torch_then_rope():
        torch_mm()
        rp.rope_partial_fwd_inplace(y, r1, r2, mode, sl)

    res = {"workload": name, "note": pw.note, "dtype": wr.dtype, "x_shape": [B, S, pw.K], "w_shape": [H * Dh, pw.K],
           "y_shape": [B, S, H, Dh], "slice": list(sl), "mode": mode, "flops_per_call": pw.flops(), "calls": {}}
    n = max(10, reps // 5)
    for label, fn in (("fused", fused), ("projection_only", plain), ("projection_then_rope", plain_then_rope),
                      ("torch_matmul_only", torch_mm), ("torch_matmul_then_rope", torch_then_rope)):
        settle(lambda j: fn(), min_launches=10, min_seconds=0.05)
        t = time_launches([(fn, ())], n, stream)
        res["calls"][label] = {"us": round(t * 1e6, 2), "TFLOPs": round(pw.flops() / t / 1e12, 1),
                               "mfma_frac": round(pw.flops() / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    del x, w, y
    torch.cuda.empty_cache()
    return res


def profile_target(name: str, reps: int, out_of_place: bool = False, positions: bool = False) -> None:
    """Launches for rocprofv3 counter passes: each direction of the workload
    `reps` times (rotating copies as in the timed run; out of place, from x
    into a second buffer; with positions, the position entry points), then a
    plain device copy of known size for calibrating the byte counters."""
    import torch

    import transformer_positional_encoding_amd as rp
    import workloads as W
    if name in W.PROJ_WORKLOADS:
        # the projection with a rotary epilogue, then the same projection with
        # an empty slice (plain GEMM)
        pw = W.PROJ_WORKLOADS[name]
        wr = W.WORKLOADS[pw.rope]
        B, S, H, Dh = pw.y_shape
        x, wt = (t.to("cuda") for t in W.make_proj_inputs(pw))
        r1, r2 = (t.to("cuda") for t in W.make_tables(wr))
        z = torch.zeros((1, 1, 1, 0), dtype=x.dtype, device="cuda")
        y = torch.empty((B, S, H, Dh), dtype=x.dtype, device="cuda")
        for _ in range(reps):
            rp.rope_proj_fwd(x, wt, r1, r2, H, wr.mode, wr.partial_slice, out=y)
        for _ in range(reps):
            rp.rope_proj_fwd(x, wt, z, z, H, wr.mode, None, out=y)
        ncopy = 1
    else:
        w = W.WORKLOADS[name]
        ncopy = 1 if out_of_place else rotating_copies(w)
        xs = [W.make_x(w).to("cuda")]
        xs += [xs[0].clone() for _ in range(ncopy - 1)]
        r1, r2 = (t.to("cuda") for t in W.make_tables(w))
        dirs = list(w.directions) + [d for d in ("fwd", "bwd") if d not in w.directions]
        y = torch.empty_like(xs[0]) if out_of_place else None
        pos = torch.from_numpy(W.positions(w)).to("cuda") if positions else None
        f = rp.rope_inv_freq(w.L, w.base, "cuda") if positions else None
        for d in dirs:
            for i in range(reps):
                if positions and out_of_place:
                    (rp.rope_partial_fwd_out_pos if d == "fwd" else rp.rope_partial_bwd_out_pos)(
                        y, xs[0], pos, f, w.mode, w.partial_slice, W.TORCH_DTYPES[w.tdtype])
                elif positions:
                    (rp.rope_partial_fwd_inplace_pos if d == "fwd" else rp.rope_partial_bwd_inplace_pos)(
                        xs[i % ncopy], pos, f, w.mode, w.partial_slice, W.TORCH_DTYPES[w.tdtype])
                elif out_of_place:
                    (rp.rope_partial_fwd_out if d == "fwd" else rp.rope_partial_bwd_out)(
                        y, xs[0], r1, r2, w.mode, w.partial_slice)
                else:
                    launch_fn(d)(xs[i % ncopy], r1, r2, w.mode, w.partial_slice)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")  # 256 MiB
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_target": name, "out_of_place": out_of_place, "positions": positions, "reps": reps,
                      "copy_bytes": src.numel(), "rotating_copies": ncopy}), flush=True)


TARGET_WORKLOADS = ("c3", "c4", "c4_f32")
PROBE_LIB = os.path.join(ROOT, "transformer_positional_encoding_amd", "_lib", "libhbm_probe.so")


def probe_fn():
    """hbm_probe_rmw from the benchmark's access-pattern probe library."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built (python -m transformer_positional_encoding_amd.build)")
    f = ctypes.CDLL(PROBE_LIB).hbm_probe_rmw
    i64 = ctypes.c_int64
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, i64, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, i64, i64,
                  ctypes.c_void_p]
    return f


def probe_variants(w) -> dict:
    """The access patterns of a workload's in-place launch, as (load range,
    store range) in 16-byte vectors of a row: the slice alone, the whole
    128-byte lines around it with the slice stored (what the rotation
    kernel loads), and the whole row (when a row is at most 64 vectors)."""
    import workloads as W
    B, S, N, D = w.x_shapes[0]
    es = W.ESIZE[w.dtype]
    row_vecs = D * es // 16
    lo, hi = w.partial_slice[0] * es, w.partial_slice[1] * es
    assert lo % 16 == 0 and hi % 16 == 0 and (D * es) % 128 == 0
    sl = (lo // 16, hi // 16)
    lines = (lo // 128 * 8, -(-hi // 128) * 8)
    out = {"slice": (sl, sl)}
    if lines != sl:
        out["lines"] = (lines, sl)
    if row_vecs <= 64:
        out["row"] = ((0, row_vecs), (0, row_vecs))
    return out


def probe_pattern(w, spec: str) -> dict:
    """One probe launch pattern from `spec` = VARIANT[:ORDER][:polK][:heads]:
    VARIANT as in probe_variants; ORDER xcd_runs (default: about 384 KiB of
    rows per XCD run, as in the rotation library), dispatch (no
    renumbering), pN (runs of N blocks) or eighth (one eighth of the grid per
    XCD); polK the load cache-policy bits K (0-7: sc0, sc1, nt; default:
    the compiler's nontemporal loads); heads: a block takes the same head of
    consecutive positions instead of consecutive heads."""
    import workloads as W
    B, S, N, D = w.x_shapes[0]
    parts = spec.split(":")
    ld, st = probe_variants(w)[parts[0]]
    span = ld[1] - ld[0]
    rpb = 64 // span
    blocks = -(-(B * S * N) // rpb)
    order, pol, stride = "xcd_runs", -1, 1
    for part in parts[1:]:
        if part.startswith("pol"):
            pol = int(part[3:])
        elif part == "heads":
            stride = N
        else:
            order = part
    if order == "xcd_runs":
        p = max(1, round((384 << 10) / (rpb * D * W.ESIZE[w.dtype])))
    elif order == "dispatch":
        p = 1
    elif order == "eighth":
        p = max(1, blocks // 8)
    else:
        p = int(order[1:])
    return {"load": ld, "store": st, "xcd_run_blocks": p, "load_policy": pol, "row_stride": stride}


# The patterns --ceiling times per workload: the slice, the kernel's whole
# lines and the whole row in two block orders; for half-line slices, every
# load cache policy; for the MLA shape, further block orders.
CEILING_PATTERNS = {
    "c4": ["slice", "slice:dispatch", "lines", "lines:dispatch", "row", "row:dispatch"]
          + [f"slice:pol{k}" for k in range(8)] + ["lines:pol4", "lines:pol0"],
    "c3": ["slice", "slice:dispatch", "row", "slice:p8", "slice:p32", "slice:p512", "slice:p2048", "slice:eighth",
           "slice:heads", "slice:heads:dispatch", "slice:pol0", "slice:pol7"],
    "c4_f32": ["slice", "slice:dispatch", "row"],
    "rh_32of128": ["slice", "slice:dispatch", "lines", "lines:dispatch", "row"],
    "rh_64of128": ["slice", "slice:dispatch", "row"],
}


def bench_ceiling(names, reps: int, stream) -> dict:
    """Each workload's bare access pattern (hbm_probe_rmw: the same bytes
    read and written back, no tables, no arithmetic) timed beside the
    rotation kernel on the same rotating copies, so each kernel can be set
    against what its access pattern alone achieves."""
    import torch

    import workloads as W
    probe = probe_fn()
    res = {}
    for name in names:
        w = W.WORKLOADS[name]
        B, S, N, D = w.x_shapes[0]
        es = W.ESIZE[w.dtype]
        rows, row_vecs = B * S * N, D * es // 16
        ncopy = rotating_copies(w)
        xs = [W.make_x(w).to("cuda")]
        xs += [xs[0].clone() for _ in range(ncopy - 1)]
        r1, r2 = (t.to("cuda") for t in W.make_tables(w))
        sptr = stream.cuda_stream
        alg = w.algorithmic_bytes()
        entry = {"x_shape": [B, S, N, D], "dtype": w.dtype, "slice": list(w.partial_slice),
                 "rotating_copies": ncopy, "algorithmic_bytes": alg, "patterns": {}}

        def probe_call(x, pat):
            rc = probe(x.data_ptr(), rows, row_vecs, pat["load"][0], pat["load"][1], pat["store"][0],
                       pat["store"][1], 1, pat["load_policy"], pat["xcd_run_blocks"], pat["row_stride"], sptr)
            if rc != 0:
                raise RuntimeError(f"hbm_probe_rmw returned {rc}")

        for _ in range(2):    # two rounds, the second kept
            for spec in CEILING_PATTERNS.get(name, ["slice", "slice:dispatch"]):
                pat = probe_pattern(w, spec)
                calls = [(probe_call, (xs[i], pat)) for i in range(ncopy)]
                time_launches(calls, max(10, reps // 2), stream)
                t = time_launches(calls, reps, stream)
                moved = rows * 2 * (pat["store"][1] - pat["store"][0]) * 16
                entry["patterns"][spec] = dict(
                    pat, avg_launch_us=round(t * 1e6, 2), slice_GBps=round(moved / t / 1e9, 1),
                    kernel_bytes_frac_at_this_time=round(alg / t / 1e9 / PEAK_GBPS, 4))
            for d in ("bwd", "fwd"):
                calls = [(launch_fn(d), (xs[i], r1, r2, w.mode, w.partial_slice)) for i in range(ncopy)]
                time_launches(calls, max(10, reps // 2), stream)
                t = time_launches(calls, reps, stream)
                entry[f"kernel_{d}_us"] = round(t * 1e6, 2)
                entry[f"kernel_{d}_frac"] = round(alg / t / 1e9 / PEAK_GBPS, 4)
        res[name] = entry
        del xs
        torch.cuda.empty_cache()
    return res


def kernel_pattern_us(name: str, reps: int, stream) -> dict:
    """The bare access pattern of the rotation kernel's in-place launch on a
    workload (the whole 128-byte lines around the slice when the slice
    covers part of a line, else the slice; the kernel's block order), timed
    as the kernel is: the ceiling its loads and stores allow."""
    import torch

    import workloads as W
    w = W.WORKLOADS[name]
    spec = "lines" if "lines" in probe_variants(w) else "slice"
    pat = probe_pattern(w, spec)
    B, S, N, D = w.x_shapes[0]
    rows, row_vecs = B * S * N, D * W.ESIZE[w.dtype] // 16
    ncopy = rotating_copies(w)
    xs = [W.make_x(w).to("cuda")]
    xs += [xs[0].clone() for _ in range(ncopy - 1)]
    probe = probe_fn()
    sptr = stream.cuda_stream

    def call(x):
        rc = probe(x.data_ptr(), rows, row_vecs, pat["load"][0], pat["load"][1], pat["store"][0], pat["store"][1],
                   1, pat["load_policy"], pat["xcd_run_blocks"], pat["row_stride"], sptr)
        if rc != 0:
            raise RuntimeError(f"hbm_probe_rmw returned {rc}")

    calls = [(call, (xs[i],)) for i in range(ncopy)]
    settle(lambda j: call(xs[j % ncopy]))
    t = time_launches(calls, reps, stream)
    del xs
    torch.cuda.empty_cache()
    return {"pattern": spec, "us": round(t * 1e6, 2),
            "frac": round(w.algorithmic_bytes() / t / 1e9 / PEAK_GBPS, 4)}


def ceiling_target(name: str, spec: str, reps: int) -> None:
    """Launches for rocprofv3 counter passes over one probe pattern (spec as
    in probe_pattern), then a device copy of known size, as profile_target
    does."""
    import torch

    import workloads as W
    w = W.WORKLOADS[name]
    B, S, N, D = w.x_shapes[0]
    rows, row_vecs = B * S * N, D * W.ESIZE[w.dtype] // 16
    pat = probe_pattern(w, spec)
    ncopy = rotating_copies(w)
    xs = [W.make_x(w).to("cuda")]
    xs += [xs[0].clone() for _ in range(ncopy - 1)]
    probe = probe_fn()
    sptr = torch.cuda.current_stream().cuda_stream
    for i in range(reps):
        rc = probe(xs[i % ncopy].data_ptr(), rows, row_vecs, pat["load"][0], pat["load"][1], pat["store"][0],
                   pat["store"][1], 1, pat["load_policy"], pat["xcd_run_blocks"], pat["row_stride"], sptr)
        if rc != 0:
            raise RuntimeError(f"hbm_probe_rmw returned {rc}")
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(pat, ceiling_target=name, spec=spec, reps=reps, copy_bytes=src.numel(),
                          rotating_copies=ncopy)), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--also", default="c3,c4_f32,c2,c4_t32,c4:out,c3:out,c4:pos,c2_s4096:pos,c3:pos,c4:outpos,"
                                      "c2_s4096:outpos,c2:posmulti,tp_qk:posmulti,c4_t32:pos,mqa_k:pos,c2_s4096,rh_64of128,"
                                      "rh_32of128,"
                                      "c3_coeff4,c3_proj",
                    help="other workloads measured in the same run (reported under 'other_workloads'); "
                         "NAME:out measures the out-of-place entry points on NAME, NAME:pos the position "
                         "entry points, NAME:outpos the out-of-place position entry points, NAME:posmulti "
                         "the multi-tensor position entry points")
    ap.add_argument("--reps", type=int, default=50, help="launches per per-kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU oracle budget: whole steps repeated to fill about this many seconds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-target", action="store_true")
    ap.add_argument("--out-of-place", action="store_true",
                    help="with --profile-target: launch the out-of-place entry points")
    ap.add_argument("--positions", action="store_true",
                    help="with --profile-target: launch the position entry points")
    ap.add_argument("--ceiling", default=None, metavar="WL,WL",
                    help="time each workload's bare access pattern (libhbm_probe.so) beside its kernel; "
                         "prints one JSON line and nothing else")
    ap.add_argument("--ceiling-target", default=None, metavar="WL:PATTERN",
                    help="launch one access pattern of the probe (for rocprofv3 counter passes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows are independent, so the operation shards over B, S or heads with no exchange "
              "between GPUs)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import transformer_positional_encoding_amd as rp
    rp.library()  # fail loudly if the HIP library is missing

    if args.profile_target:
        profile_target(args.workload, args.reps, args.out_of_place, args.positions)
        return 0
    if args.ceiling_target:
        name, _, variant = args.ceiling_target.partition(":")
        ceiling_target(name, variant, args.reps)
        return 0
    if args.ceiling:
        res = bench_ceiling([n for n in args.ceiling.split(",") if n], args.reps, torch.cuda.current_stream())
        print(json.dumps({"ceiling": res}), flush=True)
        return 0

    stream = torch.cuda.current_stream()
    main_res = bench_workload(args.workload, args.steps, args.warmup, args.reps, stream,
                              not args.no_cpu_baseline, args.cpu_seconds)
    others = []
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        import workloads as W
        if name.endswith(":out"):
            others.append(bench_out_of_place(name[:-4], args.reps, stream))
            continue
        if name.endswith(":pos"):
            others.append(bench_positions(name[:-4], args.reps, stream))
            continue
        if name.endswith(":outpos"):
            others.append(bench_positions(name[:-7], args.reps, stream, out=True))
            continue
        if name.endswith(":posmulti"):
            others.append(bench_pos_multi(name[:-9], args.reps, stream))
            continue
        if name in W.PROJ_WORKLOADS:
            others.append(bench_proj(name, args.reps, stream))
            continue
        if len(W.WORKLOADS[name].x_shapes) > 1:
            others.append(bench_multi(name, args.reps, stream))
            continue
        r = bench_workload(name, max(5, args.steps // 5), 10, args.reps, stream, False, 0)
        others.append({k: r[k] for k in ("workload", "note", "dtype", "directions", "rotating_copies",
                                         "bytes_per_launch", "elements_per_launch", "kernels")})

    import workloads as W
    w = W.WORKLOADS[args.workload]
    n_launch = len(main_res["directions"])
    step_bytes = main_res["bytes_per_launch"] * n_launch
    step_elems = main_res["elements_per_launch"] * n_launch
    value = step_bytes / main_res["step_s"] / 1e9
    dom = main_res["directions"][0]
    k = main_res["kernels"][dom]
    traffic = committed_traffic(args.workload, dom)
    roofline = {
        "bound": "hbm", "achieved": k["GBps"], "peak": PEAK_GBPS, "unit": "GB/s",
        "frac": k["frac_of_peak"],
        "traffic": None if traffic is None else traffic["hbm_bytes_per_launch"],
        "kernel": f"rope_vec_kernel ({w.dtype}, {w.mode}, {dom})",
        "bytes_per_launch": main_res["bytes_per_launch"], "avg_launch_us": k["avg_launch_us"],
    }
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_res["step_s"] * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; shapes and tables as the workload states)",
        "config": {"workload": f"{args.workload}: {w.note}", "x_shape": main_res["x_shape"],
                   "slice": main_res["slice"], "mode": w.mode, "table_shape": main_res["table_shape"],
                   "directions_per_step": main_res["directions"], "parallelism": "single GPU",
                   "rotating_copies": main_res["rotating_copies"]},
        "gelem_per_s": round(step_elems / main_res["step_s"] / 1e9, 1),
        "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
        "roofline": roofline,
        "kernels": main_res["kernels"],
        "other_workloads": "printed on the line before this one (# other_workloads ...)",
    }
    if "cpu_baseline" in main_res:
        line["cpu_baseline"] = main_res["cpu_baseline"]
    # The target: each direction of the MLA shape (c3) and the long-context
    # shard (c4, bf16 and the fp32 rerun) at >= 80% of peak HBM bandwidth in
    # algorithmic bytes. Beside each: the measured-to-algorithmic traffic
    # ratio (committed rocprofv3 counters of this kernel source) and the
    # time of the kernel's bare access pattern on this GPU.
    by_name = {main_res["workload"]: main_res}
    by_name.update({o["workload"]: o for o in others if "kernels" in o and "avg_launch_us" in
                    next(iter(o["kernels"].values()))})
    targets = {}
    for name in TARGET_WORKLOADS:
        if name not in by_name:
            continue
        ceiling = kernel_pattern_us(name, args.reps, stream)
        for d in ("fwd", "bwd"):
            k = by_name[name]["kernels"][d]
            tr = committed_traffic(name, d)
            targets[f"{name}:{d}"] = {
                "us": k["avg_launch_us"], "frac": k["frac_of_peak"], "pass": k["frac_of_peak"] >= 0.80,
                "traffic_ratio": None if tr is None else tr["traffic_over_algorithmic"],
                "pattern_us": ceiling["us"], "pattern_frac": ceiling["frac"]}
    line["targets"] = {"bar": "each direction >= 0.80 of 8 TB/s in algorithmic bytes",
                       "pattern": "the kernel's loads and stores alone (libhbm_probe), same GPU and order",
                       **targets}
    line["settle"] = dict(main_res["settle"], note="untimed launches before the warm-up: after any idle "
                          "period the first ~80 launches run 5-40% slow while the memory clocks ramp")
    # the projection with a rotary epilogue (a compact summary; the detail is
    # on the other-workloads line)
    for o in others:
        if o.get("workload") in W.PROJ_WORKLOADS:
            c = o["calls"]
            line["fused_projection"] = {
                "workload": o["workload"], "fused_us": c["fused"]["us"], "TFLOPs": c["fused"]["TFLOPs"],
                "mfma_frac": c["fused"]["mfma_frac"], "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                "projection_only_us": c["projection_only"]["us"],
                "projection_then_rope_us": c["projection_then_rope"]["us"],
                "torch_matmul_then_rope_us": c["torch_matmul_then_rope"]["us"],
                "torch_matmul_only_us": c["torch_matmul_only"]["us"]}
    # the other workloads go on a line of their own, before the result line
    print("# other_workloads " + json.dumps(others), flush=True)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
