"""ctypes binding of the C ABI in include/lse.h (argument marshalling only).

Each function has the name of the C entry point it calls and raises
``LseError`` when the status is not LSE_OK. All arithmetic runs in the HIP
library ``liblse_amd.so``; if it is missing this module raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIBRARY = Path(__file__).resolve().parent / "liblse_amd.so"

LSE_DTYPE_F32 = 0
LSE_DTYPE_BF16 = 1
LSE_DTYPE_F16 = 2

LSE_OK = 0
LSE_ERR_INVALID_ARG = 1
LSE_ERR_UNSUPPORTED_DTYPE = 2
LSE_ERR_NO_DEVICE = 3
LSE_ERR_ALLOC = 4
LSE_ERR_HIP = 5

LSE_SCHED_AUTO = 0
LSE_SCHED_ROWS_PER_WAVE = 1
LSE_SCHED_ROW_PER_WG = 2
LSE_SCHED_SPLIT_ROW = 3
SCHEDULES = {"auto": 0, "rows_per_wave": 1, "row_per_wg": 2, "split_row": 3}

LSE_SPLIT_MAX_ROWS = 1024
LSE_SPLIT_MAX_PARTS = 64

EXPORTS = ["lse_create", "lse_forward", "lse_forward_dim", "lse_token_logprob", "lse_backward",
           "lse_token_logprob_backward", "lse_backward_dim",
           "lse_destroy", "lse_status_string", "lse_set_schedule", "lse_set_tuning", "lse_plan",
           "lse_forward_noalloc"]


class LseError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class lse_plan_t(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int32), ("block", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("vector_loads", ctypes.c_int32),
                ("lanes_per_row", ctypes.c_int32), ("loads_per_lane", ctypes.c_int32),
                ("rows_per_wave", ctypes.c_int32), ("parts", ctypes.c_int32),
                ("unroll", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib: ctypes.CDLL | None = None


def load(path: Path | str = LIBRARY) -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_from(path)
    return _lib


def load_from(path: Path | str) -> ctypes.CDLL:
    """A library build at `path` with the C ABI's signatures set, loaded on its
    own (not the module's cached library): for timing two builds side by side
    (`row_wise_log_amd.ab_builds`)."""
    path = Path(path)
    if not path.exists():
        raise RuntimeError(f"{path} is missing: build it with `python -m row_wise_log_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(str(path))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "lse_create": (i32, [ctypes.POINTER(vp), ctypes.c_int]),
        "lse_forward": (i32, [vp, vp, i32, i64, i64, i64, vp, vp]),
        "lse_forward_noalloc": (i32, [vp, i32, i64, i64, i64, vp, vp]),
        "lse_token_logprob": (i32, [vp, vp, i32, i64, i64, i64, vp, vp, vp, vp]),
        "lse_backward": (i32, [vp, vp, i32, i64, i64, i64, vp, vp, vp, i64, vp]),
        "lse_token_logprob_backward": (i32, [vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, i64, vp]),
        "lse_forward_dim": (i32, [vp, vp, i32, i64, i64, i64, vp, vp]),
        "lse_backward_dim": (i32, [vp, vp, i32, i64, i64, i64, vp, vp, vp, vp]),
        "lse_destroy": (i32, [vp]),
        "lse_status_string": (ctypes.c_char_p, [i32]),
        "lse_set_schedule": (i32, [vp, i32]),
        "lse_set_tuning": (i32, [vp, i32, i32, i32, i32, i32]),
        "lse_plan": (i32, [i32, i64, i64, i64, ctypes.c_uint64, i32, i32,
                           ctypes.POINTER(lse_plan_t)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _check(status: int, where: str) -> None:
    if status != LSE_OK:
        raise LseError(status, where)


def status_string(status: int) -> str:
    return load().lse_status_string(status).decode()


lse_status_string = status_string


def lse_create(device: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(load().lse_create(ctypes.byref(h), device), "lse_create")
    return h.value


def lse_destroy(handle: int | None) -> None:
    _check(load().lse_destroy(handle), "lse_destroy")


def lse_forward(handle: int, x_ptr: int, dtype: int, rows: int, cols: int, row_stride: int,
                out_ptr: int, stream: int | None = None) -> None:
    _check(load().lse_forward(handle, x_ptr, dtype, rows, cols, row_stride, out_ptr, stream),
           "lse_forward")


def lse_forward_noalloc(x_ptr: int, dtype: int, rows: int, cols: int, row_stride: int,
                        out_ptr: int, stream: int | None = None) -> None:
    _check(load().lse_forward_noalloc(x_ptr, dtype, rows, cols, row_stride, out_ptr, stream),
           "lse_forward_noalloc")


def lse_forward_noalloc_status(x_ptr, dtype, rows, cols, row_stride, out_ptr, stream=None) -> int:
    """lse_forward_noalloc returning the raw status instead of raising (for argument tests)."""
    return load().lse_forward_noalloc(x_ptr, dtype, rows, cols, row_stride, out_ptr, stream)


def lse_forward_status(handle, x_ptr, dtype, rows, cols, row_stride, out_ptr, stream=None) -> int:
    """lse_forward returning the raw status instead of raising (for argument tests)."""
    return load().lse_forward(handle, x_ptr, dtype, rows, cols, row_stride, out_ptr, stream)


def lse_token_logprob(handle: int, x_ptr: int, dtype: int, rows: int, cols: int,
                      row_stride: int, targets_ptr: int, logp_ptr: int, lse_ptr: int | None = None,
                      stream: int | None = None) -> None:
    _check(load().lse_token_logprob(handle, x_ptr, dtype, rows, cols, row_stride, targets_ptr,
                                    logp_ptr, lse_ptr, stream), "lse_token_logprob")


def lse_token_logprob_status(handle, x_ptr, dtype, rows, cols, row_stride, targets_ptr, logp_ptr,
                             lse_ptr=None, stream=None) -> int:
    """lse_token_logprob returning the raw status instead of raising (for argument tests)."""
    return load().lse_token_logprob(handle, x_ptr, dtype, rows, cols, row_stride, targets_ptr,
                                    logp_ptr, lse_ptr, stream)


def lse_backward(handle: int, x_ptr: int, dtype: int, rows: int, cols: int, row_stride: int,
                 lse_ptr: int, grad_out_ptr: int, grad_x_ptr: int, grad_row_stride: int,
                 stream: int | None = None) -> None:
    _check(load().lse_backward(handle, x_ptr, dtype, rows, cols, row_stride, lse_ptr,
                               grad_out_ptr, grad_x_ptr, grad_row_stride, stream), "lse_backward")


def lse_token_logprob_backward(handle: int, x_ptr: int, dtype: int, rows: int, cols: int,
                               row_stride: int, targets_ptr: int, lse_ptr: int,
                               grad_logp_ptr: int, grad_x_ptr: int, grad_row_stride: int,
                               stream: int | None = None) -> None:
    _check(load().lse_token_logprob_backward(handle, x_ptr, dtype, rows, cols, row_stride,
                                             targets_ptr, lse_ptr, grad_logp_ptr, grad_x_ptr,
                                             grad_row_stride, stream),
           "lse_token_logprob_backward")


def lse_token_logprob_backward_status(handle, x_ptr, dtype, rows, cols, row_stride, targets_ptr,
                                      lse_ptr, grad_logp_ptr, grad_x_ptr, grad_row_stride,
                                      stream=None) -> int:
    """lse_token_logprob_backward returning the raw status (for argument tests)."""
    return load().lse_token_logprob_backward(handle, x_ptr, dtype, rows, cols, row_stride,
                                             targets_ptr, lse_ptr, grad_logp_ptr, grad_x_ptr,
                                             grad_row_stride, stream)


def lse_backward_status(handle, x_ptr, dtype, rows, cols, row_stride, lse_ptr, grad_out_ptr,
                        grad_x_ptr, grad_row_stride, stream=None) -> int:
    """lse_backward returning the raw status instead of raising (for argument tests)."""
    return load().lse_backward(handle, x_ptr, dtype, rows, cols, row_stride, lse_ptr,
                               grad_out_ptr, grad_x_ptr, grad_row_stride, stream)


def lse_forward_dim(handle: int, x_ptr: int, dtype: int, outer: int, n: int, inner: int,
                    out_ptr: int, stream: int | None = None) -> None:
    _check(load().lse_forward_dim(handle, x_ptr, dtype, outer, n, inner, out_ptr, stream),
           "lse_forward_dim")


def lse_forward_dim_status(handle, x_ptr, dtype, outer, n, inner, out_ptr, stream=None) -> int:
    """lse_forward_dim returning the raw status instead of raising (for argument tests)."""
    return load().lse_forward_dim(handle, x_ptr, dtype, outer, n, inner, out_ptr, stream)


def lse_backward_dim(handle: int, x_ptr: int, dtype: int, outer: int, n: int, inner: int,
                     lse_ptr: int, grad_out_ptr: int, grad_x_ptr: int,
                     stream: int | None = None) -> None:
    _check(load().lse_backward_dim(handle, x_ptr, dtype, outer, n, inner, lse_ptr, grad_out_ptr,
                                   grad_x_ptr, stream), "lse_backward_dim")


def lse_backward_dim_status(handle, x_ptr, dtype, outer, n, inner, lse_ptr, grad_out_ptr,
                            grad_x_ptr, stream=None) -> int:
    """lse_backward_dim returning the raw status instead of raising (for argument tests)."""
    return load().lse_backward_dim(handle, x_ptr, dtype, outer, n, inner, lse_ptr, grad_out_ptr,
                                   grad_x_ptr, stream)


def lse_set_schedule(handle: int, schedule: int | str) -> None:
    if isinstance(schedule, str):
        schedule = SCHEDULES[schedule]
    _check(load().lse_set_schedule(handle, schedule), "lse_set_schedule")


def lse_set_tuning(handle: int, block: int = 0, unroll: int = 0, parts: int = 0,
                   waves_per_cu: int = 0, lanes_per_row: int = 0) -> None:
    _check(load().lse_set_tuning(handle, block, unroll, parts, waves_per_cu, lanes_per_row),
           "lse_set_tuning")


def lse_plan(dtype: int, rows: int, cols: int, row_stride: int, x_addr: int = 0,
             n_cu: int = 256, schedule: int = LSE_SCHED_AUTO) -> dict:
    p = lse_plan_t()
    _check(load().lse_plan(dtype, rows, cols, row_stride, x_addr, n_cu, schedule,
                           ctypes.byref(p)), "lse_plan")
    return p.as_dict()
