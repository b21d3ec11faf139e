"""Compile the HIP library (csrc/) for gfx950 into row_wise_log_amd/liblse_amd.so.

    python -m row_wise_log_amd.build

hipcc cross-compiles for gfx950 without a GPU. Packed-fp32 VALU forms are
disabled for the device code (-packed-fp32-ops): the kernels are written with
scalar fp32 arithmetic and must compile to scalar fp32 instructions.

Kernel arguments are preloaded into scalar registers
(-amdgpu-kernarg-preload-count=16, an LLVM AMDGPU option for gfx940 and
later): a wavefront starts with its first arguments in SGPRs instead of
loading them from the kernarg segment before its first address can be formed,
one memory round trip less at the start of every launch. The code object
keeps a prologue that loads them the ordinary way, for firmware that does
not preload.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG / "liblse_amd.so"
SOURCES = [CSRC / "lse_kernels_f32.hip", CSRC / "lse_kernels_bf16.hip",
           CSRC / "lse_kernels_f16.hip", CSRC / "lse_kernels.hip", CSRC / "lse_backward.hip",
           CSRC / "lse_dim.hip", CSRC / "lse_noalloc.hip", CSRC / "lse_api.cpp"]
ARCH = "gfx950"
# The read-only control kernel that bench.py times beside the LSE kernels; its
# own library, so nothing on the LSE path can reach it.
CONTROL_LIBRARY = PKG / "libread_control.so"
CONTROL_SOURCES = [CSRC / "read_control.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(path).exists():
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")
    return path


def command(output: Path, extra: list[str] | None = None,
            sources: list[Path] | None = None) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-command-line-argument",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            f"-I{INCLUDE}", f"-I{CSRC}", *(extra or []),
            "-x", "hip", *map(str, sources or SOURCES), "-o", str(output)]


def build_control(quiet: bool = True) -> Path:
    return build(CONTROL_LIBRARY, quiet=quiet, sources=CONTROL_SOURCES)


def _report(proc: subprocess.CompletedProcess, quiet: bool) -> None:
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    if not quiet:
        # hipcc's host pass reports the device-only feature flag as unknown
        noise = "not a recognized feature for this target"
        msg = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")


def build(output: Path = LIBRARY, extra: list[str] | None = None, quiet: bool = True,
          sources: list[Path] | None = None) -> Path:
    """Compile each source to an object in parallel (one hipcc per source),
    then link the shared library; the result replaces `output` atomically."""
    sources = list(sources or SOURCES)
    tmp = output.with_name(output.name + f".tmp{os.getpid()}")
    with tempfile.TemporaryDirectory(prefix="lse_build_") as d:
        objs = [Path(d) / f"{i}_{s.stem}.o" for i, s in enumerate(sources)]
        base = command(tmp, extra, sources)
        # the compile line: the common flags, -c, one source, its object
        flags = [a for a in base[:base.index("-x")] if a != "-shared"]
        jobs = [flags + ["-c", "-x", "hip", str(s), "-o", str(o)] for s, o in zip(sources, objs)]
        workers = max(1, min(len(jobs), len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(workers) as ex:
            procs = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs))
        for proc in procs:
            _report(proc, quiet)
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs),
                "-o", str(tmp)]
        _report(subprocess.run(link, capture_output=True, text=True), quiet)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(quiet=False))
    print(build_control(quiet=False))
