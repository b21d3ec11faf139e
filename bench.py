"""Benchmark of the row-wise log-sum-exp on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--only]

One step is one lse_forward call over the whole workload: every row's
log-sum-exp in one pass. The headline workload is bf16 [512, 128256] (the
(B, N) shape the LSE paper profiles), with inputs already resident in device
memory. To measure HBM rather than the 256 MiB Infinity Cache, consecutive
steps read different copies of the input (enough copies to exceed twice the
cache), so every step streams its input from HBM.

Prints ONE JSON line with the metric, the per-launch roofline of the kernel
(algorithmic bytes / mean launch time from HIP events on the launch stream,
against the 8 TB/s HBM peak), the same-bytes read-only control kernel timed
the same way with the same launch geometry (roofline.read_control: how fast
this device reads those bytes when nothing else is done with them), and the
float64 CPU oracle's rate on the same workload as a baseline. For the forward
LSE the line also carries the other four workloads (`configs`), each timed
the same way beside its own control and checked against the oracle on every
row; --only leaves them out.

Before a workload's W warmup steps the GPU is brought to its steady state by
at least 50 ms of the control kernel's launches on the same input (which are
also the control's own timing): on a GPU that was idle, launch times move for
the first ~20 ms of continuous work, and a run with few warmup steps would
otherwise time that transient.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import workloads  # noqa: E402

METRIC = "LSE input GB/s (% of HBM peak) at [512,128256] bf16; µs/call small shapes"
METRIC_LOGPROB = "token log-prob input GB/s (x plus int64 targets) at the workload's shape"
METRIC_DIM = "LSE over the first axis input GB/s (outer 1, n rows, inner cols) at the workload's shape"
METRIC_DIM_BACKWARD = ("LSE backward over the first axis input GB/s (x, lse, grad_out read; "
                       "grad_x written) at the workload's shape")
METRIC_BACKWARD = ("LSE backward input GB/s (x, lse, grad_out read; grad_x written) at the "
                   "workload's shape")
METRIC_TOKEN_BACKWARD = ("token log-prob backward input GB/s (x, int64 targets, lse, grad_logp "
                         "read; grad_x written) at the workload's shape")
HBM_PEAK_GBS = 8000.0
CACHE_BYTES = 256 << 20
TRAFFIC_FILE = ROOT / "profiles" / "traffic.txt"
# What decides the bytes a launch moves: the kernels and the planner that picks
# the kernel instance and its grid.
KERNEL_SOURCES = [ROOT / "row_wise_log_amd" / "csrc" / n
                  for n in ("lse_kernels.h", "lse_kernels.hip", "lse_kernels_f32.hip",
                            "lse_kernels_bf16.hip", "lse_kernels_f16.hip", "lse_device.h",
                            "lse_api.cpp", "lse_launch.h")]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel and planner sources with their comments and blank
    lines removed: what decides the bytes a launch moves, not its prose."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        text = re.sub(r"/\*.*?\*/", "", p.read_text(), flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(cfg: int) -> float | None:
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; None otherwise."""
    if not TRAFFIC_FILE.exists():
        return None
    fields = {}
    for line in TRAFFIC_FILE.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_hash") != kernel_source_hash():
        return None
    v = fields.get(f"config{cfg}_bytes_per_launch")
    return float(v) if v else None


def dtype_code_of(B, dtype: str) -> int:
    return {"f32": B.LSE_DTYPE_F32, "bf16": B.LSE_DTYPE_BF16, "f16": B.LSE_DTYPE_F16}[dtype]


def host_tensor(torch, w):
    """The workload's host array as a torch tensor of its storage width."""
    return torch.from_numpy(w.x if w.dtype == "f32" else w.x.view(np.int16))


def plan_name(plan: dict) -> str:
    names = {1: "rows_per_wave", 2: "row_per_wg", 3: "split_row"}
    s = names.get(plan["schedule"], "none")
    if plan["schedule"] == 1:
        return (f"{s}(G={plan['lanes_per_row']},loads={plan['loads_per_lane']},"
                f"vec={plan['vector_loads']},grid={plan['grid']})")
    return f"{s}(block={plan['block']},unroll={plan['unroll']},parts={plan['parts']},grid={plan['grid']})"


def time_config(torch, B, handle, cfg: int, steps: int, warmup: int | None, rotate: int | None,
                op: str = "lse", graph: bool = False, w=None, extras: bool = True):
    """Time K steps of `op` on workload cfg after W warmup steps, with the
    control kernel of the same bytes timed first (its launches also bring the
    GPU to its steady state). extras: also the median of single calls and the
    graph-replayed figure."""
    w = w if w is not None else workloads.make(cfg)
    rows, cols = w.rows, w.cols
    esize = 4 if w.dtype == "f32" else 2
    in_bytes = rows * cols * esize
    out_bytes = rows * 4
    dtype_code = dtype_code_of(B, w.dtype)
    if rotate is None:
        rotate = max(1, -(-2 * CACHE_BYTES // in_bytes) + 1)
    host = host_tensor(torch, w)
    bufs = [host.to("cuda") for _ in range(rotate)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    targets = None
    bwd = None
    if op == "logprob":
        targets = torch.from_numpy(workloads.targets(cfg)).to("cuda")
        in_bytes += rows * 8  # one int64 target per row
    if op in ("backward", "logprob_backward"):
        # the forward value comes from the library's own forward pass on the
        # device (untimed), as in a training step; the oracle only checks
        lse = torch.empty(rows, dtype=torch.float32, device="cuda")
        g = np.random.default_rng(7).normal(0, 1, size=rows).astype(np.float32)
        bwd = {"lse": lse, "g": torch.from_numpy(g).to("cuda"),
               "grad": torch.empty(rows * cols, dtype=torch.float32 if w.dtype == "f32"
                                   else torch.int16, device="cuda"),
               "g_host": g}
        if op == "logprob_backward":
            bwd["targets_host"] = workloads.targets(cfg)
            bwd["targets"] = torch.from_numpy(bwd["targets_host"]).to("cuda")
            logp = torch.empty(rows, dtype=torch.float32, device="cuda")
            B.lse_token_logprob(handle, bufs[0].data_ptr(), dtype_code, rows, cols, cols,
                                bwd["targets"].data_ptr(), logp.data_ptr(), lse.data_ptr(), sh)
            in_bytes += rows * 8          # int64 targets
        else:
            B.lse_forward(handle, bufs[0].data_ptr(), dtype_code, rows, cols, cols, lse.data_ptr(), sh)
        torch.cuda.synchronize()
        bwd["lse_host"] = lse.cpu().numpy()
        out_bytes += rows * cols * esize  # grad_x
        in_bytes += rows * 8              # lse and grad_out
    if op == "dim_backward":
        # the workload's [rows, cols] array as [1, rows, cols], reduced over
        # its rows: lse from the library's own forward pass over that axis on
        # the device (untimed), one seeded incoming gradient per column
        lse = torch.empty(cols, dtype=torch.float32, device="cuda")
        B.lse_forward_dim(handle, bufs[0].data_ptr(), dtype_code, 1, rows, cols, lse.data_ptr(), sh)
        g = np.random.default_rng(7).normal(0, 1, size=cols).astype(np.float32)
        bwd = {"lse": lse, "g": torch.from_numpy(g).to("cuda"), "dim": True,
               "grad": torch.empty(rows * cols, dtype=torch.float32 if w.dtype == "f32"
                                   else torch.int16, device="cuda"),
               "g_host": g}
        torch.cuda.synchronize()
        bwd["lse_host"] = lse.cpu().numpy()
        in_bytes += cols * 8              # lse and grad_out
        out_bytes = rows * cols * esize   # grad_x
    out = torch.empty(cols if op == "dim" else rows, dtype=torch.float32, device="cuda")
    if op == "dim":
        out_bytes = cols * 4
    plan = B.lse_plan(dtype_code, rows, cols, cols, bufs[0].data_ptr(), 256, 0)

    def step(i, sh=sh):
        if op == "dim_backward":
            B.lse_backward_dim(handle, bufs[i % rotate].data_ptr(), dtype_code, 1, rows, cols,
                               bwd["lse"].data_ptr(), bwd["g"].data_ptr(), bwd["grad"].data_ptr(),
                               sh)
        elif op == "dim":
            B.lse_forward_dim(handle, bufs[i % rotate].data_ptr(), dtype_code, 1, rows, cols,
                              out.data_ptr(), sh)
        elif bwd is not None and "targets" in bwd:
            B.lse_token_logprob_backward(handle, bufs[i % rotate].data_ptr(), dtype_code, rows,
                                         cols, cols, bwd["targets"].data_ptr(),
                                         bwd["lse"].data_ptr(), bwd["g"].data_ptr(),
                                         bwd["grad"].data_ptr(), cols, sh)
        elif bwd is not None:
            B.lse_backward(handle, bufs[i % rotate].data_ptr(), dtype_code, rows, cols, cols,
                           bwd["lse"].data_ptr(), bwd["g"].data_ptr(), bwd["grad"].data_ptr(),
                           cols, sh)
        elif targets is None:
            B.lse_forward(handle, bufs[i % rotate].data_ptr(), dtype_code, rows, cols, cols,
                          out.data_ptr(), sh)
        else:
            B.lse_token_logprob(handle, bufs[i % rotate].data_ptr(), dtype_code, rows, cols, cols,
                                targets.data_ptr(), out.data_ptr(), None, sh)

    # The control first: at least PREHEAT_SECONDS of its launches (untimed),
    # then K timed ones; the LSE's warmup steps follow at once.
    nbytes = rows * cols * esize
    extra_controls = {}
    if op in ("lse", "logprob", "dim"):
        control, control_step = time_read_control(torch, bufs, nbytes, plan, steps, stream)
        if op == "lse" and plan["schedule"] == B.LSE_SCHED_ROWS_PER_WAVE and cols == 16 \
                and nbytes % 4096 == 0 and plan["lanes_per_row"] == 4:
            # many 64-byte rows: the same geometry with and without one word
            # written per row (the read + write stick the output stream needs)
            for store in (True, False):
                key = "read_write_control" if store else "read_control_same_geometry"
                extra_controls[key] = time_rows_control(torch, bufs, nbytes, int(plan["grid"]),
                                                        store, steps, stream)
    else:
        control, control_step = time_copy_control(torch, bufs, nbytes, steps, stream)
    control_step_us = control["launch_us_mean"]

    warmup = run_warmup(torch, step, warmup, stream)
    # The timed region: K back-to-back launches between a synchronize on each
    # side; the wall clock gives the whole-job rate (`value`).
    # With graph=True the K steps are captured into one HIP graph first and
    # the timed region is one replay of it (after one untimed replay).
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            hs = torch.cuda.current_stream().cuda_stream
            for i in range(steps):
                step(warmup + i, hs)
        torch.cuda.synchronize()
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            step(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The launches' own time on the GPU (`roofline.achieved`): the same K
    # steps again, with one HIP event pair on the launch stream around them,
    # queued behind a lead of control launches long enough for the host to
    # enqueue all K before the first event is reached, so the event interval
    # is the kernels' back-to-back time (plus the hardware's inter-dispatch
    # gaps) and not the host's launch rate, which short launches outrun.
    lead = max(1, int(np.ceil(steps * LEAD_US_PER_STEP / max(control_step_us, 1.0))))
    for i in range(lead):
        control_step(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            step(warmup + steps + i)
    e1.record(stream)
    torch.cuda.synchronize()
    mean_launch = e0.elapsed_time(e1) / steps
    del g

    ms_step = wall / steps * 1e3
    median_us = median_single_call_us(torch, step, warmup + 2 * steps, stream) if extras else None
    graph_us = graph_us_per_call(torch, step, warmup + 2 * steps + 60) if extras else None
    key = "frac_of_read_control" if op in ("lse", "logprob", "dim") else "frac_of_copy_control"
    control[key] = round(control["launch_us_mean"] / (mean_launch * 1e3), 4)
    for c in extra_controls.values():
        c["frac_of_control"] = round(c["launch_us_mean"] / (mean_launch * 1e3), 4)
    return {
        "w": w, "plan": plan, "rotate": rotate, "in_bytes": in_bytes, "out_bytes": out_bytes,
        "ms_per_step": ms_step, "launch_ms_mean": mean_launch,
        "value_gbs": in_bytes / (ms_step * 1e-3) / 1e9,
        "achieved_gbs": (in_bytes + out_bytes) / (mean_launch * 1e-3) / 1e9,
        "out": out, "op": op, "bwd": bwd, "control": control, "extra_controls": extra_controls,
        "median_us": median_us, "graph_us": graph_us, "warmup": warmup,
    }


WARMUP_SECONDS = 0.05


def event_mean_us(torch, step, first: int, count: int, stream) -> float:
    """Mean microseconds per launch of `count` back-to-back steps (indices
    first .. first + count - 1), one HIP event pair on `stream` around them."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(first, first + count):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / count


def run_warmup(torch, step, warmup: int | None, stream) -> int:
    """Run the untimed warmup steps and return how many ran. warmup=None
    (the default) runs at least 40 steps and at least WARMUP_SECONDS of
    back-to-back GPU work: on a GPU that was idle, launch times rise for the
    first few milliseconds of continuous work and settle after about 20 ms
    (workload 2: 22.4 -> 24.9 -> 21.9 us per launch), so a shorter warmup
    times that transient instead of the steady state."""
    if warmup is not None:
        for i in range(warmup):
            step(i)
        return warmup
    # 20 steps absorb the first call's one-time costs (code object load);
    # the next 20, timed, give the step time that sizes the rest.
    for i in range(20):
        step(i)
    per_step = max(event_mean_us(torch, step, 20, 20, stream) * 1e-6, 1e-6)
    extra = int(np.ceil(WARMUP_SECONDS / per_step))
    for i in range(40, 40 + extra):
        step(i)
    return 40 + extra


def graph_us_per_call(torch, step, first: int, calls: int = 100, replays: int = 20) -> float:
    """Microseconds per call when `calls` consecutive calls (continuing the
    input rotation) are captured into one HIP graph and the graph is
    replayed: the per-launch host and dispatch cost that a caller replaying a
    captured step sees. The entry points allocate nothing and enqueue no
    memset, so they are capturable as they are."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        hs = torch.cuda.current_stream().cuda_stream
        for i in range(calls):
            step(first + i, hs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * calls)
    del g
    return us


def median_single_call_us(torch, step, first: int, stream, calls: int = 60, skip: int = 10) -> float:
    """Median duration of single launches, each bracketed by its own event
    pair on the launch stream while the stream stays busy (the launches are
    queued back to back, so each one's start event fires when the previous
    launch ends): `calls` launches continuing the input rotation, the first
    `skip` not counted."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(first + i)
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs[skip:]]))


PREHEAT_SECONDS = 0.05
# GPU work queued ahead of the event-timed pass, per step: more than the host
# needs to enqueue one lse_forward call (a few microseconds through ctypes).
LEAD_US_PER_STEP = 15.0


def time_control(torch, step, steps: int, stream) -> float:
    """Untimed launches of a control `step` for at least PREHEAT_SECONDS of
    back-to-back GPU work (the GPU's steady state, and the control's own
    warmup), then the mean microseconds per launch of K timed ones queued
    right behind them (one HIP event pair)."""
    for i in range(5):
        step(i)
    per = max(event_mean_us(torch, step, 5, 5, stream) * 1e-6, 1e-6)
    # the untimed launches also lead the timed ones: enough GPU work for the
    # host to enqueue all K before the first event is reached
    n = max(int(np.ceil(PREHEAT_SECONDS / per)) if PREHEAT_SECONDS > 0 else 0,
            int(np.ceil(steps * LEAD_US_PER_STEP * 1e-6 / per)))
    for i in range(10, 10 + n):
        step(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(10 + n, 10 + n + steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def time_read_control(torch, bufs, nbytes: int, plan: dict, steps: int, stream) -> dict:
    """The read-only control kernel over the same input copies, in the same
    rotation, with the LSE plan's workgroup count and size: one XOR per chunk
    of the input, so the time is that of reading the bytes and nothing else.
    Timed like the LSE launches (one event pair around K back-to-back
    launches), after at least PREHEAT_SECONDS of its launches."""
    from row_wise_log_amd import read_control as RC
    grid, block = int(plan["grid"]), int(plan["block"])
    out = torch.empty(grid, dtype=torch.int32, device="cuda")
    sh = stream.cuda_stream

    def step(i):
        RC.lse_control_read(bufs[i % len(bufs)].data_ptr(), nbytes, grid, block, out.data_ptr(), sh)

    us = time_control(torch, step, steps, stream)
    return {"kernel": "read_chunks (XOR of each chunk's words)", "grid": grid, "block": block,
            "launch_us_mean": round(us, 2), "GBs": round(nbytes / (us * 1e-6) / 1e9, 1)}, step


def time_rows_control(torch, bufs, nbytes: int, grid: int, store: bool, steps: int,
                      stream) -> dict:
    """The row control on 64-byte rows with the register-rows LSE launch's
    grid: reads every row with that kernel's pattern and, with store, writes
    one 4-byte word per row with the same stores (staged in LDS, 64
    iterations at a time): the bytes the LSE launch moves, with no
    arithmetic."""
    from row_wise_log_amd import read_control as RC
    rows = nbytes // 64
    out = torch.empty(rows if store else grid * 4, dtype=torch.int32, device="cuda")
    sh = stream.cuda_stream

    def step(i):
        RC.lse_control_rows(bufs[i % len(bufs)].data_ptr(), nbytes, grid, store, out.data_ptr(), sh)

    us = time_control(torch, step, steps, stream)
    moved = nbytes + (rows * 4 if store else 0)
    return {"kernel": "rows64_chunks (XOR of each 64-byte row" +
                      (", one word stored per row)" if store else ", no stores)"),
            "grid": grid, "block": 256, "launch_us_mean": round(us, 2),
            "GBs": round(moved / (us * 1e-6) / 1e9, 1)}


def time_copy_control(torch, bufs, nbytes: int, steps: int, stream) -> dict:
    """The copy control kernel from the same input copies, in the same
    rotation, into a buffer of grad_x's size (its own, so the backward's
    output stays for the oracle check): x's bytes read and written once, one
    batch of four 16-byte vectors per lane in 256-thread workgroups (the
    backward's chunking of long rows). Timed like the backward launches."""
    from row_wise_log_amd import read_control as RC
    grid, block = -(-(nbytes // 16) // 1024), 256
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sh = stream.cuda_stream

    def step(i):
        RC.lse_control_copy(bufs[i % len(bufs)].data_ptr(), dst.data_ptr(), nbytes, grid, block, sh)

    us = time_control(torch, step, steps, stream)
    return {"kernel": "copy_chunks (x copied to a buffer of grad_x's size)", "grid": grid, "block": block,
            "launch_us_mean": round(us, 2), "GBs_read_plus_written": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}, step


def sweep_read_control(torch, cfg: int, steps: int, warmup: int) -> list:
    """The read-only control over workgroup counts 256..16384 and sizes
    256..1024 on workload cfg's input (rotating copies as in the timed
    steps); logs one JSON line per shape."""
    w = workloads.make(cfg)
    nbytes = w.x.nbytes
    host = host_tensor(torch, w)
    bufs = [host.to("cuda") for _ in range(max(1, -(-2 * CACHE_BYTES // nbytes) + 1))]
    stream = torch.cuda.current_stream()
    res = []
    for grid in (256, 512, 1024, 2048, 4096, 8192, 16384):
        for block in (256, 512, 1024):
            c, _ = time_read_control(torch, bufs, nbytes, {"grid": grid, "block": block}, steps,
                                     stream)
            rec = {"control_sweep": cfg, "grid": grid, "block": block,
                   "launch_us_mean": c["launch_us_mean"], "GBs": c["GBs"]}
            log(json.dumps(rec))
            res.append(rec)
    del bufs
    return res


def launch_floor_us(torch, B, handle, calls: int = 1000) -> float:
    """Mean time per call of 1000 back-to-back lse_forward calls on a single
    fp32 element: the library's own launch floor, beside which the small
    shapes' microseconds per call are read."""
    x = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def call(i):
        B.lse_forward(handle, x.data_ptr(), B.LSE_DTYPE_F32, 1, 1, 1, out.data_ptr(), sh)

    for i in range(50):
        call(i)
    return event_mean_us(torch, call, 50, calls, stream)


def warm_us_per_call(torch, B, handle, cfg: int, calls: int = 1000) -> float:
    """Microseconds per call of back-to-back lse_forward calls on ONE copy of
    a workload (cache-resident when it fits the 256 MiB Infinity Cache)."""
    w = workloads.make(cfg)
    x = host_tensor(torch, w).to("cuda")
    out = torch.empty(w.rows, dtype=torch.float32, device="cuda")
    code = dtype_code_of(B, w.dtype)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def call(i):
        B.lse_forward(handle, x.data_ptr(), code, w.rows, w.cols, w.cols, out.data_ptr(), sh)

    for i in range(50):
        call(i)
    return event_mean_us(torch, call, 50, calls, stream)


# Few-row shapes beside the headline: the first rows of the headline input
# (a decode step's batch of vocabulary rows) and the small fp32 workload.
SMALL_SHAPES = [("bf16", 1), ("bf16", 8), ("bf16", 32)]


def small_shapes_us(torch, B, handle, w2, calls: int = 1000) -> dict:
    """Microseconds per call of back-to-back lse_forward calls on the first 1,
    8 and 32 rows of the headline input (bf16 [r, 128256]), each call on
    another of enough copies to exceed the Infinity Cache twice, so every call
    reads HBM; with the plan the library picks for each. Returns the records
    and each shape's output of its last call (for the oracle check)."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    res, outs = {}, {}
    for dtype, rows in SMALL_SHAPES:
        x = w2.x[:rows]
        host = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        nbytes = x.nbytes
        rotate = -(-2 * CACHE_BYTES // nbytes) + 1
        big = torch.empty((rotate, rows, w2.cols), dtype=torch.int16, device="cuda")
        big[:] = host.to("cuda")
        out = torch.empty(rows, dtype=torch.float32, device="cuda")
        base, step_bytes = big.data_ptr(), nbytes

        def call(i, rows=rows):
            B.lse_forward(handle, base + (i % rotate) * step_bytes, B.LSE_DTYPE_BF16, rows, w2.cols,
                          w2.cols, out.data_ptr(), sh)

        for i in range(200):
            call(i)
        us = event_mean_us(torch, call, 200, calls, stream)
        plan = B.lse_plan(B.LSE_DTYPE_BF16, rows, w2.cols, w2.cols, base, 256, 0)
        res[f"{dtype} [{rows}, {w2.cols}]"] = {"us_per_call": round(us, 2), "plan": plan_name(plan)}
        outs[rows] = out.cpu().numpy().astype(np.float64)
        del big
    return res, outs


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.partition(":")[2].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_backward(w, r, seconds: float = 10.0) -> dict:
    """The float64 oracle's backward pass on the host cores over a bounded
    sample of rows (at most 256 MB of input); its first pass also checks the
    GPU gradient of those rows."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    orc = oracle.default()
    row_bytes = w.cols * w.x.itemsize
    n = max(1, min(w.rows, (256 << 20) // row_bytes))
    x = w.x[:n]
    lse32, g = r["bwd"]["lse_host"][:n], r["bwd"]["g_host"][:n]
    tg = r["bwd"]["targets_host"][:n] if "targets_host" in r["bwd"] else None
    passes, ref = 0, None
    t0 = time.perf_counter()
    while True:
        if tg is None:
            out = orc.softmax_grad(x, lse32, g, w.dtype, threads=threads)
        else:
            out = orc.token_logprob_grad(x, tg, lse32, g, w.dtype, threads=threads)
        if ref is None:
            ref = out
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds or passes >= 1000:
            break
    raw = r["bwd"]["grad"][: n * w.cols].cpu().numpy()
    if w.dtype == "bf16":
        got = (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    else:
        got = raw
    got = got.reshape(n, w.cols).astype(np.float64)
    fin = np.isfinite(ref)
    rel = 2.0 ** -8 + 1e-6 if w.dtype == "bf16" else 4e-7
    xv = (workloads.bf16_bits_to_f32(x) if w.dtype == "bf16" else x).astype(np.float64)
    with np.errstate(invalid="ignore"):
        d = np.abs(xv - lse32.astype(np.float64)[:, None])
    gg = np.broadcast_to(np.maximum(1.0, np.abs(g.astype(np.float64)))[:, None], ref.shape)
    if tg is None:
        tol = (rel + 2e-7 * np.where(np.isfinite(d), d, 0.0)[fin]) * np.abs(ref[fin]) + \
            2.0 ** -125 * gg[fin]
    else:
        # the softmax term's error, the added term's rounding at the target
        # column, and for bf16 one rounding of the result (as the GPU tests)
        soft = np.abs(orc.softmax_grad(x, lse32, g, w.dtype, threads=threads))
        onehot = np.zeros(ref.shape, dtype=bool)
        ok = (tg >= 0) & (tg < w.cols)
        onehot[np.arange(n)[ok], tg[ok]] = True
        dd = np.where(np.isfinite(d), d, 0.0)
        t_ = (4e-7 + 2e-7 * dd) * np.where(np.isfinite(soft), soft, 0.0) + \
            np.where(onehot, 2.0 ** -23 * np.maximum(np.abs(gg), soft), 0.0) + 2.0 ** -125 * gg
        if w.dtype == "bf16":
            t_ = t_ + (2.0 ** -8 + 1e-6) * (np.abs(np.where(np.isfinite(ref), ref, 0.0)) + t_)
        tol = t_[fin]
    err = np.abs(got[fin] - ref[fin]) / tol
    exact = bool(np.array_equal(got[~fin], ref[~fin], equal_nan=True))
    log(f"GPU gradient vs oracle ({n} rows): max |err|/tol = {err.max(initial=0):.3f}, "
        f"non-finite match {exact}")
    return {"value": round(x.nbytes * passes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "gpu_check": {"max_err_over_tol": round(float(err.max(initial=0)), 4),
                          "nonfinite_exact": exact, "rows_checked": int(n)},
            "sample": (f"the first {n} of {w.rows} rows ({x.nbytes} input bytes), {passes} passes "
                       f"in {el:.1f} s wall on {threads} threads (float64 "
                       + ("g * exp(x - lse)" if tg is None else "g * ([j == t] - exp(x - lse))")
                       + ")")}


def cpu_baseline_dim_backward(w, r, seconds: float = 10.0) -> dict:
    """The float64 oracle's backward pass over the rows axis (lse_dim_grad on
    the [1, rows, cols] array) on the host cores, over a bounded sample of
    columns (at most 256 MB of input); its first pass also checks the GPU
    gradient of those columns, at the row-wise backward pass's bar."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    esize = w.x.itemsize
    c = max(1, min(w.cols, (256 << 20) // (w.rows * esize)))
    x3 = w.x[:, :c].reshape(1, w.rows, c)
    lse32, g = r["bwd"]["lse_host"][:c], r["bwd"]["g_host"][:c]
    passes, ref = 0, None
    t0 = time.perf_counter()
    while True:
        out = oracle.lse_dim_grad(x3, lse32, g, w.dtype, threads=threads)
        if ref is None:
            ref = out[0]
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds or passes >= 1000:
            break
    raw = r["bwd"]["grad"].cpu().numpy().reshape(w.rows, w.cols)[:, :c]
    got = ((raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32) if w.dtype == "bf16"
           else raw).astype(np.float64)
    fin = np.isfinite(ref)
    rel = 2.0 ** -8 + 1e-6 if w.dtype == "bf16" else 4e-7
    xv = (workloads.bf16_bits_to_f32(x3[0]) if w.dtype == "bf16" else x3[0]).astype(np.float64)
    with np.errstate(invalid="ignore"):
        d = np.abs(xv - lse32.astype(np.float64)[None, :])
    gg = np.broadcast_to(np.maximum(1.0, np.abs(g.astype(np.float64)))[None, :], ref.shape)
    tol = (rel + 2e-7 * np.where(np.isfinite(d), d, 0.0)[fin]) * np.abs(ref[fin]) + \
        2.0 ** -125 * gg[fin]
    err = np.abs(got[fin] - ref[fin]) / tol
    exact = bool(np.array_equal(got[~fin], ref[~fin], equal_nan=True))
    log(f"GPU gradient vs oracle ({c} columns): max |err|/tol = {err.max(initial=0):.3f}, "
        f"non-finite match {exact}")
    return {"value": round(x3.nbytes * passes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "gpu_check": {"max_err_over_tol": round(float(err.max(initial=0)), 4),
                          "nonfinite_exact": exact, "columns_checked": int(c)},
            "sample": (f"the first {c} columns of the {w.rows}x{w.cols} {w.dtype} input "
                       f"({x3.nbytes} bytes), {passes} passes in {el:.1f} s wall on {threads} "
                       "threads (float64 grad_out * exp(x - lse) over a transposed copy)")}


def cpu_baseline(w, seconds: float = 10.0, op: str = "lse") -> tuple:
    """The float64 oracle on the host cores over the same input. Returns the
    baseline record and the reference (the first pass's result, with the
    LSE that scales the log-probabilities' bar) that check_gpu_output later
    holds the GPU's output of the timed steps against. bench.py runs it
    before the GPU is timed: the host works while the GPU is idle."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    orc = oracle.default()
    nbytes = w.x.nbytes
    tg = workloads.targets(w.spec.cfg) if op == "logprob" else None
    passes = 0
    t0 = time.perf_counter()
    ref = None
    while True:
        if op == "dim":
            r = oracle.lse_dim(w.x.reshape(1, w.rows, w.cols), w.dtype, threads=threads).ravel()
        elif tg is None:
            r = orc.lse(w.x, w.dtype, threads=threads)
        else:
            r = orc.token_logprob(w.x, tg, w.dtype, threads=threads)
        if ref is None:
            ref = r
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds or passes >= 1000:
            break
    lse = orc.lse(w.x, w.dtype, threads=threads) if tg is not None else None
    # one thread, over a bounded prefix of the rows (the pages time their CPU
    # LSE single-threaded)
    one = {}
    if op == "lse":
        n1 = max(1, min(w.rows, (32 << 20) // (w.cols * w.x.itemsize)))
        x1 = w.x[:n1]
        p1 = 0
        t1 = time.perf_counter()
        while True:
            orc.lse(x1, w.dtype, threads=1)
            p1 += 1
            e1 = time.perf_counter() - t1
            if e1 >= min(3.0, seconds) or p1 >= 1000:
                break
        one = {"value_1thread": round(x1.nbytes * p1 / e1 / 1e9, 3),
               "sample_1thread": f"the first {n1} rows ({x1.nbytes} bytes), {p1} passes in {e1:.1f} s"}
    rec = {"value": round(nbytes * passes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(), **one,
           "sample": (f"the whole {w.rows}x{w.cols} {w.dtype} input, {passes} passes in "
                      f"{el:.1f} s wall on {threads} threads (float64 two-pass max-subtract, "
                      "libm exp/log" + (", minus the target element" if tg is not None else "")
                      + (", over the first axis of a transposed copy" if op == "dim" else "")
                      + ")")}
    return rec, (ref, lse)


def check_gpu_output(w, gpu_out: np.ndarray, reference: tuple) -> None:
    """Hold the GPU output of the timed steps against the oracle's first pass
    (the parity bar: 2e-6 fp32, 1e-5 bf16, times max(1, |value|), and for
    log-probabilities also |LSE|; non-finite values exactly)."""
    ref, lse = reference
    tol = 2e-6 if w.dtype == "f32" else 1e-5
    fin = np.isfinite(ref)
    exact = np.array_equal(gpu_out[~fin], ref[~fin].astype(np.float32), equal_nan=True)
    scale = np.maximum(1.0, np.abs(ref[fin]))
    if lse is not None:  # logp carries the LSE's error: scale by the LSE too
        scale = np.maximum(scale, np.abs(lse[fin]))
    err = np.abs(gpu_out[fin] - ref[fin]) / (tol * scale)
    log(f"GPU output vs oracle: max |err|/tol = {err.max(initial=0):.3f}, non-finite match {exact}")
    return {"max_err_over_tol": round(float(err.max(initial=0)), 4), "nonfinite_exact": bool(exact),
            "rows_checked": int(len(ref))}


def oracle_reference(w, op: str = "lse"):
    """The float64 oracle over every output of the workload, on all host
    cores (the checker of the timed steps' output; not timed as a baseline),
    as (reference, LSE for the log-probabilities' bar); None for the backward
    ops, whose outputs the backward baseline checks on the headline only."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    if op == "lse":
        return oracle.lse(w.x, w.dtype, threads=threads), None
    if op == "logprob":
        lse = oracle.lse(w.x, w.dtype, threads=threads)
        return oracle.token_logprob(w.x, workloads.targets(w.spec.cfg), w.dtype, threads=threads), lse
    if op == "dim":
        return oracle.lse_dim(w.x.reshape(1, w.rows, w.cols), w.dtype, threads=threads).ravel(), None
    return None


def torch_context(torch, w, steps: int) -> dict:
    """The pages' own comparison on this input: torch.logsumexp and torch.sum
    over the last axis of the same device tensor (the paper's section 1 sets
    one against the other; its Figure 1 profiles the former's sub-kernels at
    this shape), mean microseconds per call over K calls cycling through
    copies larger than the Infinity Cache. Context only: never on the
    library's path."""
    host = torch.from_numpy(w.x.view(np.int16))
    nb = w.x.nbytes
    rotate = max(1, -(-2 * CACHE_BYTES // nb) + 1)
    bufs = [host.to("cuda").view(torch.bfloat16) if w.dtype == "bf16" else host.to("cuda")
            for _ in range(rotate)]
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in (("torch.logsumexp", lambda t: torch.logsumexp(t, dim=1)),
                     ("torch.sum", lambda t: torch.sum(t, dim=1))):
        def call(i, fn=fn):
            fn(bufs[i % rotate])
        for i in range(10):
            call(i)
        res[name + "_us"] = round(event_mean_us(torch, call, 10, max(steps, 20), stream), 2)
    del bufs
    res["note"] = (f"on the same {w.dtype} device tensor, dim=1, torch {torch.__version__}; "
                   "the pages report 1.95 ms against 0.31 ms on another GPU (context only)")
    return res


def reduced_bit_context(torch, B, handle, steps: int, warmup: int | None) -> dict:
    """The paper's reduced-bit comparison (§4.3, Figure 5: FuseLSE16 against
    FuseLSE) on this GPU, at the headline shape: the same seeded fp32 values
    stored as fp32, bf16 and fp16, each timed like the headline (its control
    first, then W warmup and K timed steps) and its output checked two ways:
    against the oracle on its own stored bits (the parity bar), and against
    the float64 LSE of the unrounded fp32 values (the error that storing the
    input in 16 bits costs, the quantity the paper's MAE measures)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    base = workloads.make(2, storage="f32")
    exact = oracle.lse(base.x, "f32", threads=threads)
    res = {}
    for storage in ("f32", "bf16", "f16"):
        wc = base if storage == "f32" else workloads.make(2, storage=storage)
        log(f"reduced-bit context: the headline values stored as {storage}")
        rc = time_config(torch, B, handle, 2, steps, warmup, None, "lse", w=wc, extras=False)
        got = rc["out"].cpu().numpy().astype(np.float64)
        chk = check_gpu_output(wc, got, (oracle.lse(wc.x, storage, threads=threads), None))
        dev = np.abs(got - exact)
        res[storage] = {"us_per_launch": round(rc["launch_ms_mean"] * 1e3, 2),
                        "input_bytes": rc["in_bytes"],
                        "achieved_GBs": round(rc["achieved_gbs"], 1),
                        "mae_vs_f64_of_fp32_values": float(f"{dev.mean():.3g}"),
                        "max_abs_err_vs_f64_of_fp32_values": float(f"{dev.max():.3g}"),
                        "max_err_over_tol_own_bits": chk["max_err_over_tol"]}
        del rc, wc
    for storage in ("bf16", "f16"):
        res[storage]["speedup_over_f32"] = round(
            res["f32"]["us_per_launch"] / res[storage]["us_per_launch"], 3)
    res["note"] = ("the paper reports FuseLSE16 at 12.06x and FuseLSE at 6.25x over "
                   "torch.logsumexp with FuseLSE16's mean absolute error below 3e-3 (another GPU); "
                   "here the 16-bit formats halve the bytes read and the arithmetic stays fp32")
    return res


def versions(torch) -> dict:
    rocm = "unknown"
    try:
        rocm = Path("/opt/rocm/.info/version").read_text().strip()
    except OSError:
        pass
    return {"numpy": np.__version__, "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None), "rocm": rocm}


def config_record(r: dict, check: dict | None, traffic: float | None) -> dict:
    """The compact record of one workload for the `configs` key."""
    w = r["w"]
    us = r["launch_ms_mean"] * 1e3
    forward = r["op"] in ("lse", "logprob", "dim")
    rec = {"workload": f"config{w.spec.cfg} {w.spec.name}: {w.spec.recipe}",
           "rows": w.rows, "cols": w.cols, "input_dtype": w.dtype, "op": r["op"],
           "plan": plan_name(r["plan"]) if r["op"] in ("lse", "logprob") else f"lse_{r['op']}",
           "us_per_launch": round(us, 2),
           "us_per_call_wall": round(r["ms_per_step"] * 1e3, 2),
           "input_GBs_wall": round(r["value_gbs"], 1),
           "rows_per_s": round(w.rows / (r["ms_per_step"] * 1e-3), 1),
           "algorithmic_bytes_per_launch": r["in_bytes"] + r["out_bytes"],
           "achieved_GBs": round(r["achieved_gbs"], 1),
           "frac_of_hbm_peak": round(r["achieved_gbs"] / HBM_PEAK_GBS, 4),
           "traffic": traffic,
           ("read_control" if forward else "copy_control"): r["control"],
           "warmup": r["warmup"]}
    rec.update(r["extra_controls"])
    if check is not None:
        rec.update(check)
    return rec


# ---- plan A/B at the steady state ---------------------------------------------

def parse_plan(spec: str) -> dict:
    """'auto' or comma-separated key=value with keys schedule (auto,
    rows_per_wave, row_per_wg, split_row), block, unroll, parts, waves_per_cu,
    lanes_per_row: a plan forced through lse_set_schedule / lse_set_tuning."""
    plan = {"schedule": "auto", "block": 0, "unroll": 0, "parts": 0, "waves_per_cu": 0,
            "lanes_per_row": 0}
    if spec.strip() != "auto":
        for item in spec.split(","):
            k, _, v = item.partition("=")
            k = k.strip()
            if k not in plan:
                raise SystemExit(f"unknown plan key {k!r} in {spec!r}")
            plan[k] = v.strip() if k == "schedule" else int(v)
    return plan


def plan_ab(torch, B, dtype: str, rows: int, cols: int, plans: list, blocks: int = 4,
            block_ms: float = 30.0, warm_ms: float = 100.0) -> dict:
    """Alternate blocks of back-to-back lse_forward launches of each plan on
    one shape (random N(0, 3^2) rows, rotating copies beyond the Infinity
    Cache) after warm_ms of launches: each block runs at least block_ms, one
    event pair around it; the median over the blocks of each plan's mean
    microseconds per launch. Every plan's output is checked against the
    float64 oracle."""
    import oracle
    rng = np.random.default_rng(rows * 7 + cols)
    v = rng.normal(0, 3, size=(rows, cols)).astype(np.float32)
    x = v if dtype == "f32" else (workloads.f32_to_bf16_bits(v) if dtype == "bf16"
                                   else workloads.f32_to_f16_bits(v))
    del v
    ref = oracle.lse(x, dtype, threads=len(os.sched_getaffinity(0)))
    nbytes = x.nbytes
    rotate = max(1, -(-2 * CACHE_BYTES // nbytes) + 1)
    host = torch.from_numpy(x if dtype == "f32" else x.view(np.int16))
    bufs = [host.to("cuda") for _ in range(rotate)]
    code = dtype_code_of(B, dtype)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    handles, outs = [], []
    for pl in plans:
        h = B.lse_create(0)
        B.lse_set_schedule(h, pl["schedule"])
        B.lse_set_tuning(h, pl["block"], pl["unroll"], pl["parts"], pl["waves_per_cu"],
                         pl["lanes_per_row"])
        handles.append(h)
        outs.append(torch.empty(rows, dtype=torch.float32, device="cuda"))

    def step_of(j):
        h, o = handles[j], outs[j]
        return lambda i: B.lse_forward(h, bufs[i % rotate].data_ptr(), code, rows, cols, cols,
                                       o.data_ptr(), sh)

    steps = [step_of(j) for j in range(len(plans))]
    checks = []
    for j, st in enumerate(steps):
        st(0)
        torch.cuda.synchronize()
        checks.append(check_gpu_output(type("W", (), {"dtype": dtype})(),
                                       outs[j].cpu().numpy().astype(np.float64), (ref, None)))
    per = [max(event_mean_us(torch, st, 0, 10, stream), 0.5) for st in steps]
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < warm_ms * 1e-3:
        steps[i % len(steps)](i)
        i += 1
    means = [[] for _ in plans]
    for _ in range(blocks):
        for j, st in enumerate(steps):
            n = max(20, int(np.ceil(block_ms * 1e3 / per[j])))
            means[j].append(event_mean_us(torch, st, 0, n, stream))
    plan_info = []
    for pl in plans:
        pi = B.lse_plan(code, rows, cols, cols, bufs[0].data_ptr(), 256, B.SCHEDULES[pl["schedule"]])
        for k in ("block", "unroll", "parts"):  # the forced tuning overrides the planner's
            if pl[k] and pi["schedule"] != 1:
                pi[k] = pl[k]
        if pl["parts"] and pi["schedule"] == 3:
            pi["grid"] = min(rows, B.LSE_SPLIT_MAX_ROWS) * pl["parts"]
        plan_info.append(pi)
    for h in handles:
        B.lse_destroy(h)
    med = [float(np.median(m)) for m in means]
    return {"dtype": dtype, "rows": rows, "cols": cols, "bytes": nbytes,
            "plans": [{"forced": pl, "planned": plan_name(pi), "us_median": round(m, 2),
                       "us_blocks": [round(u, 2) for u in ms], **ck}
                      for pl, pi, m, ms, ck in zip(plans, plan_info, med, means, checks)],
            "ratio_b_over_a": round(med[1] / med[0], 4) if len(med) > 1 else None}


# ---- rocprofv3 summaries (no GPU needed) ------------------------------------
#
# The summaries under profiles/ are written by these functions from the CSV
# files that `rocprofv3 ... --output-format csv -d DIR -o run -- python3
# bench.py ...` leaves in DIR, so that each one can be regenerated from
# committed code.

def _csv_rows(directory: str, suffix: str) -> list:
    import csv
    rows = []
    for f in sorted(Path(directory).rglob(f"*{suffix}")):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def short_kernel_name(name: str) -> str:
    name = name.strip()
    return name[:name.index("(", name.index(">"))] if ">" in name and "(" in name else name


def summarize_trace(directory: str) -> str:
    """Markdown table of a kernel trace: per kernel, dispatches and the mean,
    median, min and max duration in microseconds."""
    groups: dict[tuple, list] = {}
    for r in _csv_rows(directory, "kernel_trace.csv"):
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        block = int(r["Workgroup_Size_X"])
        key = (short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(block, 1), block)
        groups.setdefault(key, []).append(us)
    out = ["| kernel | workgroups x threads | dispatches | mean us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for (name, wgs, block), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(v)
        out.append(f"| `{name}` | {wgs} x {block} | {len(a)} | {a.mean():.2f} | {np.median(a):.2f} | "
                   f"{a.min():.2f} | {a.max():.2f} |")
    return "\n".join(out)


def summarize_trace_runs(directory: str, min_len: int = 50) -> str:
    """Markdown table of the runs in a kernel trace: maximal sequences of
    consecutive dispatches (in dispatch order) of one kernel and launch shape,
    at least min_len long, e.g. one workload's warmup and timed steps."""
    rows = sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Dispatch_Id"]))
    runs, cur, key0 = [], [], None
    for r in rows:
        block = int(r["Workgroup_Size_X"])
        key = (short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(block, 1), block)
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        if key != key0 and cur:
            runs.append((key0, int(cur[0][0]), cur))
            cur = []
        key0 = key
        cur.append((r["Dispatch_Id"], us))
    if cur:
        runs.append((key0, int(cur[0][0]), cur))
    out = ["| first dispatch | kernel | workgroups x threads | dispatches | mean us | mean of the last "
           "1000 us | median us |", "|---|---|---|---|---|---|---|"]
    for (name, wgs, block), first, v in runs:
        if len(v) < min_len:
            continue
        a = np.array([u for _, u in v])
        out.append(f"| {first} | `{name}` | {wgs} x {block} | {len(a)} | {a.mean():.2f} | "
                   f"{a[-1000:].mean():.2f} | {np.median(a):.2f} |")
    return "\n".join(out)


CONTROL_KERNELS = ("read_chunks", "copy_chunks", "rows64_chunks")


def summarize_event_passes(directory: str, steps: int = 1000) -> str:
    """Markdown table of the event-timed passes in a kernel trace of bench.py.
    bench.py runs a workload's warmup and wall-clock launches, then a lead of
    control launches, then the event-timed launches of the same kernel: so a
    run of a library kernel whose previous run is a control kernel and whose
    run before that is the same kernel and launch shape is an event pass, and
    its first `steps` dispatches are the timed launches. Reported with their
    span (first start to last end, per dispatch: the interval an event pair
    around them measures, gaps included) and the mean of the control's lead
    run."""
    rows = sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Dispatch_Id"]))
    runs, cur, key0 = [], [], None
    for r in rows:
        block = int(r["Workgroup_Size_X"])
        key = (short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(block, 1), block)
        if key != key0 and cur:
            runs.append((key0, cur))
            cur = []
        key0 = key
        cur.append((int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3,
                    int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    if cur:
        runs.append((key0, cur))
    out = ["| first dispatch | kernel | workgroups x threads | timed dispatches | mean us | min us | max us | "
           "span per dispatch us | control lead before it: dispatches, mean us |",
           "|---|---|---|---|---|---|---|---|---|"]
    for (k2, _), (k1, lead), (key, v) in zip(runs, runs[1:], runs[2:]):
        if k2 != key or "lse::" not in key[0] or not any(c in k1[0] for c in CONTROL_KERNELS):
            continue
        timed = v[:steps]
        a = np.array([e[1] for e in timed])
        c = np.array([e[1] for e in lead])
        # first start to last end over the dispatches: what an event pair around them measures
        span = (timed[-1][3] - timed[0][2]) * 1e-3 / len(timed)
        out.append(f"| {v[0][0]} | `{key[0]}` | {key[1]} x {key[2]} | {len(a)} | {a.mean():.2f} | "
                   f"{a.min():.2f} | {a.max():.2f} | {span:.2f} | {len(c)}, {c.mean():.2f} |")
    return "\n".join(out)


def counter_means(directory: str) -> dict:
    """{kernel: {counter: mean value per dispatch}} from a counter collection."""
    acc: dict[str, dict[str, list]] = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        k = short_kernel_name(r["Kernel_Name"])
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: (float(np.mean(v)), len(v)) for c, v in d.items()} for k, d in acc.items()}


def summarize_counters(directory: str) -> str:
    """Markdown table: per kernel and counter, the mean per dispatch."""
    out = ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for k, d in sorted(counter_means(directory).items()):
        for c, (m, n) in sorted(d.items()):
            out.append(f"| `{k}` | {c} | {n} | {m:.6g} |")
    return "\n".join(out)


def plan_kernel_name(plan: dict, dtype: str, cols: int) -> str:
    """The demangled name of the kernel instance an lse_forward plan launches."""
    d = {"f32": 0, "bf16": 1, "f16": 2}[dtype]
    if plan["schedule"] == 1:
        vpl, g, vec = plan["loads_per_lane"], plan["lanes_per_row"], plan["vector_loads"]
        rounds = 4 if vpl == 1 else (2 if vpl == 2 else 1)
        k = (4 if dtype == "f32" else 8) if vec else 1
        tail = bool(vec) and cols % k != 0
        return (f"void lse::rows_in_registers<(lse::DType){d}, {g}, {vpl}, {str(bool(vec)).lower()}, "
                f"{str(tail).lower()}, {rounds}, false>")
    split = "true" if plan["schedule"] == 3 else "false"
    return f"void lse::stream_rows<(lse::DType){d}, {plan['block']}, {plan['unroll']}, {split}, false>"


def write_traffic(fetch_dir: str, write_dir: str, copy_bytes: int, command: str) -> str:
    """profiles/traffic.txt from a FETCH_SIZE run and a WRITE_SIZE run of the
    default forward bench (all five workloads), each counter scaled by
    known / measured for the three plain device copies of copy_bytes bytes the
    bench makes first (the copy kernel's dispatches)."""
    from row_wise_log_amd import binding as B
    fetch, write = counter_means(fetch_dir), counter_means(write_dir)

    def factor(directory, counter):
        # the calibration copies are the first three copy-kernel dispatches
        rows = [r for r in _csv_rows(directory, "counter_collection.csv")
                if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        if len(rows) < 3:
            raise SystemExit(f"fewer than three copy-kernel dispatches with {counter}")
        measured = float(np.mean([float(r["Counter_Value"]) for r in rows[:3]]))
        return (copy_bytes / 1024.0) / measured

    ff, fw = factor(fetch_dir, "FETCH_SIZE"), factor(write_dir, "WRITE_SIZE")
    lines = ["# HBM traffic per launch from rocprofv3 counters (read by bench.py for roofline.traffic).",
             "# FETCH_SIZE / WRITE_SIZE means (KiB per dispatch) scaled by known/measured for the three",
             f"# plain device copies of {copy_bytes} bytes the bench makes first in the same process.",
             "# Commands (from the repository root, one counter per run):",
             f"#   {command.replace('COUNTER', 'FETCH_SIZE')}",
             f"#   {command.replace('COUNTER', 'WRITE_SIZE')}",
             "# then: python3 bench.py --write-traffic FETCH_DIR WRITE_DIR --copy-bytes "
             f"{copy_bytes}",
             "# bench.py reports roofline.traffic only while kernel_source_hash matches the sources.",
             f"kernel_source_hash: {kernel_source_hash()}"]
    for cfg in (1, 2, 3, 4, 5):
        spec = workloads.SPECS[cfg]
        esize = 4 if spec.dtype == "f32" else 2
        plan = B.lse_plan(dtype_code_of(B, spec.dtype), spec.rows, spec.cols, spec.cols, 0, 256, 0)
        k = plan_kernel_name(plan, spec.dtype, spec.cols)
        if k not in fetch or k not in write:
            raise SystemExit(f"config {cfg}: kernel {k} not in the counter runs")
        fkib, wkib = fetch[k]["FETCH_SIZE"][0], write[k]["WRITE_SIZE"][0]
        total = fkib * 1024 * ff + wkib * 1024 * fw
        alg = spec.rows * spec.cols * esize + 4 * spec.rows
        lines.append(f"# config {cfg}: {k}: FETCH {fkib:.1f} KiB x {ff:.4f}, WRITE {wkib:.1f} KiB x "
                     f"{fw:.4f}; algorithmic {spec.rows * spec.cols * esize} + {4 * spec.rows} B; "
                     f"traffic/algorithmic = {total / alg:.4f}")
        lines.append(f"config{cfg}_bytes_per_launch: {total:.0f}")
    return "\n".join(lines) + "\n"


def main() -> int:
    global PREHEAT_SECONDS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least 40 steps and at least 50 ms of "
                         "back-to-back GPU work); the control kernel's launches run before them")
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--rotate", type=int, default=None,
                    help="input copies cycled through (default: enough to exceed 2x the 256 MiB cache)")
    ap.add_argument("--all", action="store_true",
                    help="also time the other four workloads for --op logprob, backward, "
                         "logprob_backward or dim (the forward LSE line carries them by default)")
    ap.add_argument("--only", action="store_true",
                    help="time only the --config workload (the forward LSE line otherwise also "
                         "carries the other four workloads under `configs`)")
    ap.add_argument("--no-small-shapes", action="store_true",
                    help="leave out the few-row shapes of the headline input (counter runs that "
                         "select the headline kernel by name)")
    ap.add_argument("--no-torch-context", action="store_true",
                    help="leave out torch.logsumexp / torch.sum on the headline tensor")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--op", choices=["lse", "logprob", "backward", "logprob_backward", "dim",
                                     "dim_backward"],
                    default="lse",
                    help="lse: lse_forward (the headline); logprob: lse_token_logprob with one "
                         "seeded int64 target per row; backward: lse_backward (reads x, writes "
                         "grad_x) on the forward pass's own LSE; logprob_backward: "
                         "lse_token_logprob_backward (the same, with the targets); dim: "
                         "lse_forward_dim over the workload's first axis")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps into one HIP graph and time one replay of it "
                         "(the same K full calls on the same rotating inputs; default: K eager "
                         "launches)")
    ap.add_argument("--control-sweep", action="store_true",
                    help="also time the read-only control kernel over a grid of workgroup counts "
                         "and sizes on the workload's input, one JSON line each to stderr (is "
                         "any launch shape a faster way to read these bytes?)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run three plain device copies of BYTES bytes (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--preheat-seconds", type=float, default=0.05,
                    help="minimum duration of each workload's untimed control launches before its "
                         "warmup steps (0 in counter runs, where launches are serialised)")
    ap.add_argument("--ab", nargs=3, action="append", metavar=("DTYPE", "ROWS", "COLS"),
                    help="plan A/B on a shape (repeatable): alternate blocks of --plan launches "
                         "at the steady state and print one JSON line per shape, then exit")
    ap.add_argument("--plan", action="append", default=None,
                    help="a plan for --ab: 'auto' or e.g. 'schedule=row_per_wg,block=256' (give two "
                         "or more; default: auto against row_per_wg)")
    ap.add_argument("--ab-blocks", type=int, default=4)
    ap.add_argument("--ab-block-ms", type=float, default=30.0)
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 kernel trace (CSV) and exit: per "
                         "kernel, per run of consecutive dispatches, and the event-timed passes "
                         "(their first --steps dispatches)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 counter collection and exit")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.txt from a FETCH_SIZE and a WRITE_SIZE run and exit")
    ap.add_argument("--copy-bytes", type=int, default=268435456,
                    help="size of the calibration copies in the counter runs (--write-traffic)")
    ap.add_argument("--traffic-command", default=(
        "rocprofv3 --pmc COUNTER --output-format csv -d <dir> -o run -- python3 bench.py "
        "--no-cpu-baseline --no-torch-context --steps 5 --warmup 1 --preheat-seconds 0 "
        "--copy-calibration 268435456"))
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        print()
        print(summarize_trace_runs(args.summarize_trace))
        print()
        print(summarize_event_passes(args.summarize_trace, args.steps))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return 0
    if args.write_traffic:
        TRAFFIC_FILE.write_text(write_traffic(*args.write_traffic, args.copy_bytes,
                                              args.traffic_command))
        print(TRAFFIC_FILE.read_text())
        return 0

    PREHEAT_SECONDS = args.preheat_seconds

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the row-wise LSE "
                                   "shards by rows with no communication, so --gpus N > 1 is "
                                   "not measured here"}))
        return 2

    import torch

    from row_wise_log_amd import binding as B
    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    B.load()
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration: 3 copies of {args.copy_calibration} bytes")
        del src, dst
    if args.ab:
        plans = [parse_plan(p_) for p_ in (args.plan or ["auto", "schedule=row_per_wg"])]
        for dt, rows_, cols_ in args.ab:
            res = plan_ab(torch, B, dt, int(rows_), int(cols_), plans, args.ab_blocks,
                          args.ab_block_ms)
            print(json.dumps(res), flush=True)
        return 0
    handle = B.lse_create(0)
    try:
        log(f"timing config {args.config} ({args.op}): {args.steps} steps after "
            f"{'at least 50 ms of' if args.warmup is None else args.warmup} warmup")
        # The forward ops' CPU baseline runs first, while the GPU is idle; its
        # reference checks the timed steps' output afterwards. (The backward
        # baselines need the timed run's inputs and run after it.)
        w0, reference = None, None
        early = not args.no_cpu_baseline and args.op in ("lse", "logprob", "dim")
        if early:
            w0 = workloads.make(args.config)
            log("timing the float64 oracle on the host cores")
            cpu_rec, reference = cpu_baseline(w0, args.cpu_seconds, args.op)
        r = time_config(torch, B, handle, args.config, args.steps, args.warmup, args.rotate,
                        args.op, args.graph, w=w0)
        w = r["w"]
        traffic = recorded_traffic(args.config) if args.op == "lse" else None
        floor = launch_floor_us(torch, B, handle)
        log(f"launch floor (lse_forward on one element, back to back): {floor:.2f} us per call")
        small = small_out = None
        if args.op == "lse" and args.config == 2 and not args.graph and not args.no_small_shapes:
            small, small_out = small_shapes_us(torch, B, handle, w)
            log(f"few-row shapes: {small}")
        line = {
            "metric": {"lse": METRIC, "logprob": METRIC_LOGPROB, "backward": METRIC_BACKWARD,
                       "logprob_backward": METRIC_TOKEN_BACKWARD,
                       "dim": METRIC_DIM, "dim_backward": METRIC_DIM_BACKWARD}[args.op],
            "value": round(r["value_gbs"], 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": r["warmup"],
            "ms_per_step": round(r["ms_per_step"], 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f32",
            "data": "synthetic",
            "config": {
                "workload": f"config{args.config} {w.spec.name}: {w.spec.recipe}",
                "rows": w.rows, "cols": w.cols, "input_dtype": w.dtype,
                "op": args.op,
                "input_bytes": r["in_bytes"], "output_bytes": r["out_bytes"],
                "rotating_copies": r["rotate"],
                "plan": plan_name(r["plan"]) if args.op in ("lse", "logprob") else f"lse_{args.op}",
                "pct_of_hbm_peak": round(100 * r["value_gbs"] / HBM_PEAK_GBS, 2),
                "us_per_call": round(r["ms_per_step"] * 1e3, 2),
                "rows_per_s": round(w.rows / (r["ms_per_step"] * 1e-3), 1),
                "launch_floor_us": round(floor, 2),
                "graph_us_per_call": round(r["graph_us"], 2),
                "timed_as": "one HIP graph replay of the K steps" if args.graph
                            else "K eager launches",
                "preheat": "at least 50 ms of the control kernel's launches on the same input "
                           "right before the warmup steps",
                "input_sha256": workloads.sha256(w.x),
            },
            "roofline": {
                "bound": "hbm",
                "achieved": round(r["achieved_gbs"], 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(r["achieved_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "launch_us_mean": round(r["launch_ms_mean"] * 1e3, 2),
                "launch_us_median_single_calls": round(r["median_us"], 2),
                "algorithmic_bytes_per_launch": r["in_bytes"] + r["out_bytes"],
                ("read_control" if args.op in ("lse", "logprob", "dim") else "copy_control"):
                    r["control"],
                **r["extra_controls"],
            },
            "versions": versions(torch),
        }
        if args.op == "lse" and args.config == 2 and not args.no_torch_context:
            ctx = torch_context(torch, w, args.steps)
            ctx["speedup_of_lse_forward_over_torch_logsumexp"] = round(
                ctx["torch.logsumexp_us"] / (r["launch_ms_mean"] * 1e3), 2)
            line["torch_context"] = ctx
            log(f"torch context: {ctx}")
        if args.op == "lse" and args.config == 2 and not args.only:
            line["reduced_bit"] = reduced_bit_context(torch, B, handle, args.steps, args.warmup)
            log(f"reduced-bit context: {line['reduced_bit']}")
        if args.control_sweep:
            sweep_read_control(torch, args.config, args.steps, r["warmup"])
        if early:
            chk = check_gpu_output(w, r["out"].cpu().numpy().astype(np.float64), reference)
            line.update(chk)
            if small_out:  # the few-row shapes are the headline input's first rows
                for rows, got in small_out.items():
                    log(f"first {rows} rows:")
                    small[f"bf16 [{rows}, {w.cols}]"].update(
                        check_gpu_output(w, got, (reference[0][:rows], None)))
            line["cpu_baseline"] = cpu_rec
        elif not args.no_cpu_baseline:
            log("timing the float64 oracle on the host cores")
            line["cpu_baseline"] = (cpu_baseline_dim_backward(w, r, args.cpu_seconds)
                                    if args.op == "dim_backward"
                                    else cpu_baseline_backward(w, r, args.cpu_seconds))
        else:
            line["cpu_baseline"] = None
        if small is not None:
            line["small_shapes"] = small
        del r
        if (args.op == "lse" and not args.only) or args.all:
            # The other four workloads: each timed the same way (its control
            # first, then W warmup and K timed steps) and, for the forward
            # ops, checked on every row.
            others = {}
            for cfg in [c for c in (1, 2, 3, 4, 5) if c != args.config]:
                wc = workloads.make(cfg)
                log(f"timing config {cfg} ({args.op})")
                rc = time_config(torch, B, handle, cfg, args.steps, args.warmup, None, args.op,
                                 args.graph, w=wc, extras=False)
                ref = oracle_reference(wc, args.op)
                chk = None
                if ref is not None:
                    chk = check_gpu_output(wc, rc["out"].cpu().numpy().astype(np.float64), ref)
                rec = config_record(rc, chk, recorded_traffic(cfg) if args.op == "lse" else None)
                if cfg == 1 and args.op == "lse":
                    rec["us_per_call_warm"] = round(warm_us_per_call(torch, B, handle, cfg), 2)
                log(json.dumps(rec))
                others[str(cfg)] = rec
                del rc, wc, ref
                torch.cuda.empty_cache()
            line["configs"] = others
        print(json.dumps(line), flush=True)
    finally:
        torch.cuda.synchronize()
        B.lse_destroy(handle)
    return 0


if __name__ == "__main__":
    sys.exit(main())
