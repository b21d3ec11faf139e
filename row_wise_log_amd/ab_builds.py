"""Time two or more builds of the library against each other on the same
inputs (the "library copies" behind the planner and kernel comments).

    python -m row_wise_log_amd.ab_builds --lib base.so --lib new.so[:PARTS] \\
        [--forward bf16:512:128256] [--dim bf16:512:50257] [--dim-backward f32:65536:4097] \\
        [--blocks 6] [--block-ms 30]

A build is any `liblse_amd.so` compiled from these sources with a change
(`python -m row_wise_log_amd.build` writes the in-tree one; copy it aside
before rebuilding); `:PARTS` forces `lse_set_tuning`'s parts on that build's
handle. Shapes are DTYPE:ROWS:COLS: `--forward` reduces each row
(lse_forward), `--dim` and `--dim-backward` take the array as [1, ROWS, COLS]
and reduce over ROWS (lse_forward_dim, lse_backward_dim with lse from the
first build's forward and seeded N(0, 1) grad_out).

Per shape: seeded N(0, 3) values in copies enough to exceed twice the
256 MiB Infinity Cache (calls rotate through them); every build runs once
and its output is compared with the first build's (bit for bit, and the
largest relative difference over finite outputs); then `blocks` rounds time
each build in turn for about `block_ms` ms of calls behind a lead of the
same build's calls (HIP events on the current stream), and the median of
each build's block means is printed, beside a control kernel over the same
bytes (a read for the forward ops, a copy for the backward) from the in-tree
control library. Needs a GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import statistics
import time
from pathlib import Path

from . import binding as B
from . import read_control as RC

CACHE_BYTES = 256 << 20
DTYPES = {"f32": 0, "bf16": 1, "f16": 2}


def parse_shape(spec: str) -> tuple[str, int, int]:
    """DTYPE:ROWS:COLS with DTYPE one of f32, bf16, f16."""
    parts = spec.split(":")
    if len(parts) != 3 or parts[0] not in DTYPES:
        raise argparse.ArgumentTypeError(f"shape {spec!r}: want DTYPE:ROWS:COLS, DTYPE in {sorted(DTYPES)}")
    rows, cols = int(parts[1]), int(parts[2])
    if rows <= 0 or cols <= 0:
        raise argparse.ArgumentTypeError(f"shape {spec!r}: sizes must be positive")
    return parts[0], rows, cols


def parse_lib(spec: str) -> tuple[Path, int]:
    """PATH or PATH:PARTS."""
    path, sep, parts = spec.rpartition(":")
    if sep and parts.isdigit():
        return Path(path), int(parts)
    return Path(spec), 0


def rotation(nbytes: int) -> int:
    """Copies of an input so that the rotation exceeds twice the cache."""
    return min(4096, max(1, -(-2 * CACHE_BYTES // nbytes) + 1))


def _timed(torch, steps, stream, blocks: int, block_ms: float) -> list[list[float]]:
    def ev_mean(step, n, lead):
        for i in range(lead):
            step(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    per = [max(ev_mean(st, 10, 0), 0.5) for st in steps]
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < 0.1:
        steps[i % len(steps)](i)
        i += 1
    means = [[] for _ in steps]
    for _ in range(blocks):
        for j, st in enumerate(steps):
            n = max(20, int(block_ms * 1e3 / per[j]) + 1)
            means[j].append(ev_mean(st, n, min(int(n * 15 / per[j]) + 1, 2000)))
    return means


def run_shape(torch, op: str, shape, libs, blocks: int, block_ms: float) -> None:
    dtype, rows, cols = shape
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    code = DTYPES[dtype]
    g = torch.Generator().manual_seed(rows * 1000003 + cols)
    host = (torch.randn(rows, cols, generator=g) * 3).to(tdt)
    nbytes = host.numel() * host.element_size()
    pitch = -(-nbytes // 256) * 256
    copies = rotation(nbytes)
    buf = torch.empty(copies * pitch, dtype=torch.uint8, device="cuda")
    flat = host.view(-1).view(torch.uint8).cuda()
    for c in range(copies):
        buf[c * pitch: c * pitch + nbytes] = flat
    base = buf.data_ptr()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    out_len = {"forward": rows, "dim": cols, "dim-backward": rows * cols}[op]
    out_dt = tdt if op == "dim-backward" else torch.float32
    handles, outs, steps = [], [], []
    lse = gout = None
    if op == "dim-backward":
        lib0, _ = libs[0]
        h0 = ctypes.c_void_p()
        assert lib0.lse_create(ctypes.byref(h0), 0) == 0
        lse = torch.empty(cols, dtype=torch.float32, device="cuda")
        assert lib0.lse_forward_dim(h0, base, code, 1, rows, cols, lse.data_ptr(), sh) == 0
        torch.cuda.synchronize()
        lib0.lse_destroy(h0)
        gout = torch.randn(cols, generator=g).cuda()
    for lib, parts in libs:
        h = ctypes.c_void_p()
        assert lib.lse_create(ctypes.byref(h), 0) == 0
        if parts:
            assert lib.lse_set_tuning(h, 0, 0, parts, 0, 0) == 0
        o = torch.empty(out_len, dtype=out_dt, device="cuda")
        handles.append((lib, h))
        outs.append(o)

        def step(i, lib=lib, h=h, o=o):
            x = base + (i % copies) * pitch
            if op == "forward":
                rc = lib.lse_forward(h, x, code, rows, cols, cols, o.data_ptr(), sh)
            elif op == "dim":
                rc = lib.lse_forward_dim(h, x, code, 1, rows, cols, o.data_ptr(), sh)
            else:
                rc = lib.lse_backward_dim(h, x, code, 1, rows, cols, lse.data_ptr(), gout.data_ptr(),
                                          o.data_ptr(), sh)
            if rc != 0:
                raise RuntimeError(f"{op} {shape}: status {rc}")
        steps.append(step)
    names = [f"build{j}" for j in range(len(libs))]
    if nbytes % 16 == 0:  # the control kernels take whole 16-byte words
        chunks = max(1, nbytes // 16384)
        if op == "dim-backward":
            dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            steps.append(lambda i: RC.lse_control_copy(base + (i % copies) * pitch, dst.data_ptr(),
                                                       nbytes, chunks, 256, sh))
            names.append("copy_control")
        else:
            red = torch.empty(chunks, dtype=torch.int32, device="cuda")
            steps.append(lambda i: RC.lse_control_read(base + (i % copies) * pitch, nbytes, chunks,
                                                       256, red.data_ptr(), sh))
            names.append("read_control")
    for st in steps:
        st(0)
    torch.cuda.synchronize()
    ref = outs[0].float().double()
    fin = torch.isfinite(ref)
    print(f"{op} {dtype} [{rows}, {cols}]", flush=True)
    for j in range(1, len(libs)):
        same = torch.equal(outs[0].view(torch.uint8), outs[j].view(torch.uint8))
        got = outs[j].float().double()
        rel = ((got - ref).abs() / ref.abs().clamp(min=1.0))[fin]
        worst = rel.max().item() if rel.numel() else 0.0
        nonfin = torch.equal(torch.isfinite(got), fin)
        print(f"   {names[j]} against build0: bitwise {same}, max rel diff {worst:.3g}, "
              f"non-finite pattern equal {nonfin}", flush=True)
    means = _timed(torch, steps, stream, blocks, block_ms)
    for nm, ms in zip(names, means):
        print(f"   {nm:13s} median {statistics.median(ms):9.2f} us   blocks {[round(u, 2) for u in ms]}",
              flush=True)
    for lib, h in handles:
        lib.lse_destroy(h)
    del buf
    torch.cuda.empty_cache()


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--lib", action="append", type=parse_lib, required=True,
                    help="a library build, PATH or PATH:PARTS (at least two; the first is the reference)")
    ap.add_argument("--forward", action="append", type=parse_shape, default=[])
    ap.add_argument("--dim", action="append", type=parse_shape, default=[])
    ap.add_argument("--dim-backward", action="append", type=parse_shape, default=[])
    ap.add_argument("--blocks", type=int, default=6)
    ap.add_argument("--block-ms", type=float, default=30.0)
    a = ap.parse_args(argv)
    if len(a.lib) < 2:
        ap.error("give at least two --lib builds")
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("ab_builds needs a GPU")
    libs = [(B.load_from(path), parts) for path, parts in a.lib]
    for i, (path, parts) in enumerate(a.lib):
        print(f"build{i}: {path}" + (f" (parts {parts})" if parts else ""), flush=True)
    for op, shapes in (("forward", a.forward), ("dim", a.dim), ("dim-backward", a.dim_backward)):
        for shape in shapes:
            run_shape(torch, op, shape, libs, a.blocks, a.block_ms)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
