"""ctypes binding of the control kernels (csrc/read_control.hip).

The read control reads a byte range once, with the streaming LSE schedule's
loads and pipeline, and keeps only the XOR of each chunk's 32-bit words; the
copy control reads a range and writes it to another buffer the same way; the
row control reads 64-byte rows with the register-rows schedule's pattern and
optionally writes one word per row (the read + write stick for many short
rows).
bench.py times them on the same buffers and launch geometry as an LSE launch
(read) or a backward launch (copy), which shows how far each kernel sits from
plainly moving the same bytes on the same device. They are measurement
infrastructure: they live in their own library and the LSE entry points never
call them.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIBRARY = Path(__file__).resolve().parent / "libread_control.so"

_lib: ctypes.CDLL | None = None


def load(path: Path | str = LIBRARY) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = Path(path)
    if not path.exists():
        raise RuntimeError(f"{path} is missing: build it with `python -m row_wise_log_amd.build`")
    lib = ctypes.CDLL(str(path))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.lse_control_read.restype = ctypes.c_int
    lib.lse_control_read.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp]
    lib.lse_control_copy.restype = ctypes.c_int
    lib.lse_control_copy.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp]
    lib.lse_control_rows.restype = ctypes.c_int
    lib.lse_control_rows.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp]
    _lib = lib
    return lib


def lse_control_read(x: int, nbytes: int, chunks: int, block: int, out: int, stream: int) -> None:
    """XOR of the 32-bit words of each of `chunks` pieces of x[0:nbytes] into
    out[chunks] (device pointers; x 16-byte aligned, nbytes a multiple of 16)."""
    rc = load().lse_control_read(x, nbytes, chunks, block, out, stream)
    if rc == 1:
        raise ValueError(f"lse_control_read: invalid argument (bytes={nbytes}, chunks={chunks}, "
                         f"block={block})")
    if rc != 0:
        raise RuntimeError(f"lse_control_read: launch failed ({rc})")


def lse_control_copy(src: int, dst: int, nbytes: int, chunks: int, block: int, stream: int) -> None:
    """Copy src[0:nbytes] to dst (device pointers, 16-byte aligned, not
    overlapping; nbytes a multiple of 16) in `chunks` workgroups of `block`."""
    rc = load().lse_control_copy(src, dst, nbytes, chunks, block, stream)
    if rc == 1:
        raise ValueError(f"lse_control_copy: invalid argument (bytes={nbytes}, chunks={chunks}, "
                         f"block={block})")
    if rc != 0:
        raise RuntimeError(f"lse_control_copy: launch failed ({rc})")


def lse_control_rows(x: int, nbytes: int, grid: int, store: bool, out: int, stream: int) -> None:
    """Read x[0:nbytes] as 64-byte rows with the register-rows LSE pattern
    (`grid` workgroups of 256 threads); with store, write each row's XOR to
    out[row] (nbytes / 64 words), else one XOR per wavefront to out[wave]
    (grid * 4 words). x 16-byte aligned, nbytes a multiple of 4096."""
    rc = load().lse_control_rows(x, nbytes, grid, 1 if store else 0, out, stream)
    if rc == 1:
        raise ValueError(f"lse_control_rows: invalid argument (bytes={nbytes}, grid={grid})")
    if rc != 0:
        raise RuntimeError(f"lse_control_rows: launch failed ({rc})")
