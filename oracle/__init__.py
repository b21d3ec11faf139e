"""float64 CPU oracle for the row-wise log-sum-exp.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers. The HIP library never
imports, links or runs anything here, and this package imports nothing from
it.

``lse(x, dtype)`` returns, for each row of a 2-D array, log(sum_j exp(x_ij))
in float64, computed by ``lse_oracle.c`` (plain two-pass max-subtract with
libm ``exp``/``log``; its header states the definition and the special
cases). ``token_logprob(x, targets, dtype)`` returns x[r, targets[r]] minus
that LSE (NaN for a target outside [0, cols)); ``softmax_grad(x, lse, g,
dtype)`` returns the backward pass g[r] * exp(x[r, j] - lse[r]) in float64;
``token_logprob_grad(x, targets, lse, g, dtype)`` returns the token
log-probability's backward pass g[r] * ([j == t_r] - exp(x[r, j] - lse[r]));
``lse_dim(x3, dtype)`` reduces the middle axis of an [outer, n, inner] array
(torch.logsumexp over a non-last axis) by moving that axis last and calling
the row oracle.
bf16 inputs are passed as uint16 bit patterns; fp16 inputs as float16 arrays or
their uint16 bit patterns with dtype "f16".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "lse_oracle.c"
LIBRARY = HERE / "liblse_oracle.so"

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}


def build(source: Path = SOURCE, output: Path = LIBRARY) -> Path:
    """Compile the oracle with gcc: -O2, IEEE semantics (no fast-math)."""
    tmp = output.with_name(output.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Werror", "-pthread",
           "-o", str(tmp), str(source), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


class Oracle:
    """ctypes view of one compiled oracle library (the real one, or a test mutant)."""

    def __init__(self, path: Path = LIBRARY):
        path = Path(path)
        if not path.exists():
            build(output=path)
        self.path = path
        self._lib = ctypes.CDLL(str(path))
        fn = self._lib.lse_oracle_f64
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        self._fn = fn
        fn = self._lib.lse_oracle_token_logprob_f64
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        self._fn_tok = fn
        fn = self._lib.lse_oracle_softmax_grad_f64
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_int]
        self._fn_grad = fn
        fn = self._lib.lse_oracle_token_logprob_grad_f64
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_int]
        self._fn_tok_grad = fn

    def softmax_grad(self, x: np.ndarray, lse, grad_out, dtype: str | None = None,
                     threads: int = 1) -> np.ndarray:
        """grad_out[r] * exp(x[r, j] - lse[r]) in float64, shape (rows, cols);
        lse and grad_out are taken as fp32, as a caller of the backward pass holds them."""
        x, dtype, rows, cols, stride = self._prepare(x, dtype)
        lse = np.ascontiguousarray(np.asarray(lse, dtype=np.float32))
        g = np.ascontiguousarray(np.asarray(grad_out, dtype=np.float32))
        if lse.shape != (rows,) or g.shape != (rows,):
            raise ValueError("lse and grad_out must hold one value per row")
        out = np.full((rows, cols), np.nan, dtype=np.float64)
        rc = self._fn_grad(x.ctypes.data if x.size else None, DTYPES[dtype], rows, cols, stride,
                           lse.ctypes.data if rows else None, g.ctypes.data if rows else None,
                           out.ctypes.data, int(threads))
        if rc != 0:
            raise ValueError("lse_oracle_softmax_grad_f64 rejected its arguments")
        return out

    def token_logprob_grad(self, x: np.ndarray, targets, lse, grad_logp,
                           dtype: str | None = None, threads: int = 1) -> np.ndarray:
        """grad_logp[r] * ([j == t_r] - exp(x[r, j] - lse[r])) in float64, shape
        (rows, cols); a row of NaN for a target outside [0, cols). lse and
        grad_logp are taken as fp32."""
        x, dtype, rows, cols, stride = self._prepare(x, dtype)
        t = np.ascontiguousarray(np.asarray(targets, dtype=np.int64))
        lse = np.ascontiguousarray(np.asarray(lse, dtype=np.float32))
        g = np.ascontiguousarray(np.asarray(grad_logp, dtype=np.float32))
        if t.shape != (rows,) or lse.shape != (rows,) or g.shape != (rows,):
            raise ValueError("targets, lse and grad_logp must hold one value per row")
        out = np.full((rows, cols), np.nan, dtype=np.float64)
        rc = self._fn_tok_grad(x.ctypes.data if x.size else None, DTYPES[dtype], rows, cols,
                               stride, t.ctypes.data if rows else None,
                               lse.ctypes.data if rows else None, g.ctypes.data if rows else None,
                               out.ctypes.data, int(threads))
        if rc != 0:
            raise ValueError("lse_oracle_token_logprob_grad_f64 rejected its arguments")
        return out

    @staticmethod
    def _prepare(x: np.ndarray, dtype: str | None):
        x = np.asarray(x)
        if dtype is None:
            dtype = {np.dtype(np.uint16): "bf16", np.dtype(np.float16): "f16"}.get(x.dtype, "f32")
        if dtype == "f16" and x.dtype == np.float16:
            x = x.view(np.uint16)  # fp16 is passed as its bit patterns
        want = np.float32 if dtype == "f32" else np.uint16
        if x.dtype != want:
            raise TypeError(f"dtype {dtype} needs a {np.dtype(want)} array, got {x.dtype}")
        if x.ndim != 2:
            raise ValueError("x must be 2-D")
        rows, cols = x.shape
        if (cols > 1 and x.strides[1] != x.itemsize) or \
                (rows > 1 and (x.strides[0] < cols * x.itemsize or x.strides[0] % x.itemsize)):
            x = np.ascontiguousarray(x)
        stride = x.strides[0] // x.itemsize if rows > 1 else cols
        return x, dtype, rows, cols, stride

    def token_logprob(self, x: np.ndarray, targets, dtype: str | None = None,
                      threads: int = 1) -> np.ndarray:
        """x[r, targets[r]] - LSE(x[r, :]) in float64 (NaN for a target outside [0, cols))."""
        x, dtype, rows, cols, stride = self._prepare(x, dtype)
        t = np.ascontiguousarray(np.asarray(targets, dtype=np.int64))
        if t.shape != (rows,):
            raise ValueError("targets must hold one int64 per row")
        out = np.full(rows, np.nan, dtype=np.float64)
        rc = self._fn_tok(x.ctypes.data if x.size else None, DTYPES[dtype], rows, cols, stride,
                          t.ctypes.data if rows else None, out.ctypes.data, int(threads))
        if rc != 0:
            raise ValueError("lse_oracle_token_logprob_f64 rejected its arguments")
        return out

    def lse(self, x: np.ndarray, dtype: str | None = None, threads: int = 1) -> np.ndarray:
        """Row-wise LSE of a 2-D array in float64.

        ``x`` is float32 (dtype "f32"), uint16 bf16 bits (dtype "bf16"), or
        float16 / uint16 fp16 bits (dtype "f16"; a float16 array implies it).
        Any row stride is accepted as long as the last axis is contiguous.
        """
        x, dtype, rows, cols, stride = self._prepare(x, dtype)
        out = np.full(rows, np.nan, dtype=np.float64)  # rows left unwritten stay NaN
        rc = self._fn(x.ctypes.data if x.size else None, DTYPES[dtype], rows, cols,
                      stride, out.ctypes.data, int(threads))
        if rc != 0:
            raise ValueError("lse_oracle_f64 rejected its arguments")
        return out

    def raw(self, ptr, dtype_code: int, rows: int, cols: int, stride: int, out_ptr,
            threads: int = 1) -> int:
        """Direct call with raw pointers, for argument-checking tests."""
        return self._fn(ptr, dtype_code, rows, cols, stride, out_ptr, threads)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def lse(x: np.ndarray, dtype: str | None = None, threads: int = 1) -> np.ndarray:
    return default().lse(x, dtype, threads)


def token_logprob(x: np.ndarray, targets, dtype: str | None = None, threads: int = 1) -> np.ndarray:
    return default().token_logprob(x, targets, dtype, threads)


def softmax_grad(x: np.ndarray, lse, grad_out, dtype: str | None = None,
                 threads: int = 1) -> np.ndarray:
    return default().softmax_grad(x, lse, grad_out, dtype, threads)


def token_logprob_grad(x: np.ndarray, targets, lse, grad_logp, dtype: str | None = None,
                       threads: int = 1) -> np.ndarray:
    return default().token_logprob_grad(x, targets, lse, grad_logp, dtype, threads)


def lse_dim(x3: np.ndarray, dtype: str | None = None, threads: int = 1) -> np.ndarray:
    """LSE over the middle axis of an [outer, n, inner] array, float64 [outer, inner].

    The plain definition: the same log-sum-exp, over a different axis. The
    reduced axis is moved last (a transposed copy) and each (o, i) is one row
    of the row oracle. The paper presents its kernels as drop-in replacements
    for torch.logsumexp, whose `dim` may be any axis (abstract, §6).
    """
    x3 = np.asarray(x3)
    if x3.ndim != 3:
        raise ValueError("x3 must be 3-D [outer, n, inner]")
    outer, n, inner = x3.shape
    rows = np.ascontiguousarray(np.transpose(x3, (0, 2, 1))).reshape(outer * inner, n)
    return default().lse(rows, dtype, threads).reshape(outer, inner)



def lse_dim_grad(x3: np.ndarray, lse2, grad_out2, dtype: str | None = None,
                 threads: int = 1) -> np.ndarray:
    """The backward of lse_dim: grad[o, j, i] = grad_out[o, i] * exp(x[o, j, i] - lse[o, i])
    in float64 for an [outer, n, inner] array, with lse and grad_out [outer, inner]
    (fp32 values as the GPU receives them).

    The plain definition: the row oracle's softmax_grad (whose formula is pinned by
    finite differences) over a different axis. The reduced axis is moved last (a
    transposed copy), each (o, i) is one row with its own lse and grad_out, and the
    result is moved back. The paper lists backward support for its kernels (Table 3)
    and offers them as drop-in replacements for torch.logsumexp over any axis
    (abstract, §6).
    """
    x3 = np.asarray(x3)
    if x3.ndim != 3:
        raise ValueError("x3 must be 3-D [outer, n, inner]")
    outer, n, inner = x3.shape
    lse2 = np.asarray(lse2, dtype=np.float32).reshape(outer * inner)
    g2 = np.asarray(grad_out2, dtype=np.float32).reshape(outer * inner)
    rows = np.ascontiguousarray(np.transpose(x3, (0, 2, 1))).reshape(outer * inner, n)
    g = default().softmax_grad(rows, lse2, g2, dtype, threads=threads)
    return np.ascontiguousarray(np.transpose(g.reshape(outer, inner, n), (0, 2, 1)))
