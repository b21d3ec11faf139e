"""Row-wise log-sum-exp on MI355X (gfx950): a C-ABI HIP library and its binding.

``logsumexp(x)`` returns log(sum(exp(x), dim=-1)) in fp32 for a 2-D fp32,
bf16 or fp16 CUDA/HIP tensor whose last axis is contiguous; ``logsumexp_autograd(x)``
is the same value with a gradient (the library's backward pass, grad_out *
exp(x - lse), in x's dtype); ``logsumexp_dim(x, d)`` reduces any axis of a
contiguous tensor (``logsumexp_dim_autograd`` with its gradient);
``token_logprob(x, t)`` returns x[r, t[r]] - logsumexp(x)[r] from the same
single pass. The plain helpers turn into their autograd variants when x
requires a gradient. PyTorch only provides the device memory and the current
stream; the computation is the HIP library's ``lse_forward`` /
``lse_backward`` / ``lse_forward_dim`` / ``lse_backward_dim`` /
``lse_token_logprob`` / ``lse_token_logprob_backward`` (see include/lse.h);
``token_logprob_autograd(x, t)`` is the token log-probability with its
gradient. The library is loaded on first use
and a missing library is an error, never a fallback. The helpers keep one
library handle per (device, stream); ``prepare(stream)`` makes it ahead of a
HIP graph capture on that stream (none can be made during one), and
``release()`` frees handles.
"""
from __future__ import annotations

import threading
from collections import OrderedDict

from .binding import (LseError, lse_create, lse_destroy, lse_forward,  # noqa: F401
                      lse_forward_noalloc, lse_plan, lse_set_schedule, lse_set_tuning,
                      lse_status_string, lse_token_logprob, load)

# Library handles of the torch helpers, one per (device, stream): a handle's
# split workspace must not serve two streams at once, and calls on one stream
# are ordered, so they can share one. Handles are created outside graph
# capture only (lse_create allocates and synchronises). At most
# MAX_HANDLES_PER_DEVICE unpinned handles are kept per device, the least
# recently used one released beyond that (after a device synchronisation);
# handles made by prepare(), or used while a stream was being captured (a
# captured graph keeps their workspace addresses), are pinned and live until
# release().
MAX_HANDLES_PER_DEVICE = 8
_handles: OrderedDict[tuple[int, int], int] = OrderedDict()
_pinned: set[tuple[int, int]] = set()
# Guards _handles and _pinned: helpers called from several host threads (one
# stream each) must neither make two handles for one key nor evict a handle
# another thread has just looked up.
_lock = threading.RLock()


def _capturing() -> bool:
    import torch

    return torch.cuda.is_current_stream_capturing()


def _evict(device: int) -> None:
    import torch

    loose = [k for k in _handles if k[0] == device and k not in _pinned]
    if len(loose) < MAX_HANDLES_PER_DEVICE:
        return
    torch.cuda.synchronize(device)  # no work may still use the handle
    for key in loose[:len(loose) - MAX_HANDLES_PER_DEVICE + 1]:
        lse_destroy(_handles.pop(key))


def handle(device: int, stream: int = 0) -> int:
    """The library handle for `device` and the stream handle `stream`. Made
    on first use, outside graph capture; under capture a stream with no
    handle yet is an error (call prepare() for it before capturing)."""
    key = (device, int(stream))
    capturing = _capturing()
    with _lock:
        h = _handles.get(key)
        if h is None:
            if capturing:
                raise RuntimeError(
                    "row_wise_log_amd: no library handle for this stream, and one cannot be made "
                    "while the stream is being captured (lse_create allocates and synchronises); "
                    "call row_wise_log_amd.prepare(stream) before the capture")
            _evict(device)
            h = lse_create(device)
            _handles[key] = h
        else:
            _handles.move_to_end(key)
        if capturing:
            _pinned.add(key)
        return h


def prepare(stream=None, device: int | None = None) -> int:
    """Make (outside graph capture) and pin the handle that the helpers use
    on `stream` (a torch.cuda.Stream or a raw stream handle; default the
    current stream of `device`, default the current device). Call it before
    capturing helpers into a HIP graph on that stream. Returns the handle."""
    import torch

    if _capturing():
        raise RuntimeError("row_wise_log_amd.prepare() must run outside graph capture")
    if device is None:
        device = stream.device.index if isinstance(stream, torch.cuda.Stream) else \
            torch.cuda.current_device()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    raw = stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)
    with _lock:
        h = handle(device, raw)
        _pinned.add((device, raw))
        return h


def release(stream=None, device: int | None = None) -> None:
    """Release the helpers' handles (pinned ones included): the one of
    `stream` if given, else every handle of `device`, else all. Synchronises
    the devices concerned first; graphs captured with those handles must not
    be replayed afterwards."""
    import torch

    with _lock:
        if stream is not None:
            raw = stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)
            keys = [k for k in _handles if k[1] == raw and (device is None or k[0] == device)]
        else:
            keys = [k for k in _handles if device is None or k[0] == device]
        for d in sorted({k[0] for k in keys}):
            torch.cuda.synchronize(d)
        for k in keys:
            _pinned.discard(k)
            lse_destroy(_handles.pop(k))


def _device_stream(x) -> tuple[int, int]:
    import torch

    return x.device.index or 0, torch.cuda.current_stream(x.device).cuda_stream


def _dtype_codes(torch) -> dict:
    from .binding import LSE_DTYPE_BF16, LSE_DTYPE_F16, LSE_DTYPE_F32

    return {torch.float32: LSE_DTYPE_F32, torch.bfloat16: LSE_DTYPE_BF16,
            torch.float16: LSE_DTYPE_F16}


def _check_input(x):
    import torch

    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows, cols)")
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    codes = _dtype_codes(torch)
    if x.dtype not in codes:
        raise TypeError(f"unsupported dtype {x.dtype}: fp32, bf16 or fp16")
    rows, cols = x.shape
    if cols > 1 and x.stride(1) != 1:
        raise ValueError("the last axis must be contiguous")
    return codes[x.dtype], rows, cols, (x.stride(0) if rows > 1 else cols)


def _dim_geometry(x, dim, keepdim: bool):
    """(outer, n, inner, output shape) of torch.logsumexp(x, dim, keepdim) for a
    contiguous tensor: the reduced axes (one, or a tuple of adjacent ones) form n."""
    import torch

    if x.dim() == 0:
        raise ValueError("x must have at least one axis")
    nd = x.dim()
    raw = list(dim) if isinstance(dim, (tuple, list)) else [dim]
    if not raw:
        raise ValueError("dim must name at least one axis")
    for d in raw:
        if not -nd <= d < nd:
            raise IndexError(f"dim {d} is out of range for a {nd}-D tensor")
    dims = sorted(d % nd for d in raw)
    if len(set(dims)) != len(dims):
        raise ValueError(f"dim {tuple(raw)} names an axis more than once")
    if dims != list(range(dims[0], dims[-1] + 1)):
        raise NotImplementedError("the reduced axes must be adjacent")
    codes = _dtype_codes(torch)
    if x.dtype not in codes:
        raise TypeError(f"unsupported dtype {x.dtype}: fp32, bf16 or fp16")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    d0, d1 = dims[0], dims[-1]
    shape = list(x.shape)
    outer = 1
    for s_ in shape[:d0]:
        outer *= s_
    n = 1
    for s_ in shape[d0:d1 + 1]:
        n *= s_
    inner = 1
    for s_ in shape[d1 + 1:]:
        inner *= s_
    kept = shape[:d0] + ([1] * (d1 - d0 + 1) if keepdim else []) + shape[d1 + 1:]
    return outer, n, inner, kept


def logsumexp_dim(x, dim, keepdim: bool = False, handle_=None):
    """LSE over axis `dim` of a contiguous fp32/bf16/fp16 GPU tensor of any rank, as
    fp32 (torch.logsumexp(x, dim, keepdim) semantics). `dim` may also be a
    tuple of adjacent axes, which a contiguous tensor holds as one axis; other
    tuples raise NotImplementedError. When x requires a gradient (and grad mode
    is on) this is logsumexp_dim_autograd: the same value, differentiable
    through the library's backward pass."""
    import torch

    from .binding import lse_forward_dim

    if _needs_grad(torch, x):
        if handle_ is not None:
            raise RuntimeError("logsumexp_dim(): handle_ does not support automatic "
                               "differentiation, and x requires grad")
        return logsumexp_dim_autograd(x, dim, keepdim)
    outer, n, inner, kept = _dim_geometry(x, dim, keepdim)
    out = torch.empty(kept, dtype=torch.float32, device=x.device)
    dev, stream = _device_stream(x)
    h = handle_ if handle_ is not None else handle(dev, stream)
    lse_forward_dim(h, x.data_ptr(), _dtype_codes(torch)[x.dtype], outer, n, inner,
                    out.data_ptr(), stream)
    return out


def _dim_autograd_function():
    import torch

    from .binding import lse_backward_dim

    class _LogSumExpDim(torch.autograd.Function):
        """LSE over any axis with the library's backward pass (lse_backward_dim)."""

        @staticmethod
        def forward(ctx, x, dim, keepdim):
            out = logsumexp_dim(x, dim, keepdim)
            ctx.save_for_backward(x, out)
            ctx.geometry = _dim_geometry(x, dim, keepdim)[:3]
            return out

        @staticmethod
        def backward(ctx, grad_out):
            x, out = ctx.saved_tensors
            outer, n, inner = ctx.geometry
            g = grad_out.to(torch.float32).contiguous()
            lse = out.contiguous()
            grad = torch.empty_like(x)
            dev, stream = _device_stream(x)
            h = handle(dev, stream)
            lse_backward_dim(h, x.data_ptr(), _dtype_codes(torch)[x.dtype], outer, n, inner,
                             lse.data_ptr(), g.data_ptr(), grad.data_ptr(), stream)
            return grad, None, None

    return _LogSumExpDim


_LSE_DIM_FN = None


def logsumexp_dim_autograd(x, dim, keepdim: bool = False):
    """logsumexp_dim with a gradient: with respect to x it is grad_out *
    exp(x - lse) broadcast along the reduced axes (each column's softmax along
    them, scaled by its incoming gradient), computed by the library's
    lse_backward_dim and returned in x's dtype."""
    global _LSE_DIM_FN
    if _LSE_DIM_FN is None:
        _LSE_DIM_FN = _dim_autograd_function()
    return _LSE_DIM_FN.apply(x, dim, keepdim)


def _needs_grad(torch, x) -> bool:
    return x.requires_grad and torch.is_grad_enabled()


def logsumexp(x, out=None, handle_=None):
    """LSE over the last axis of a 2-D fp32/bf16/fp16 GPU tensor, as fp32[rows].
    When x requires a gradient (and grad mode is on) this is logsumexp_autograd,
    as torch.logsumexp would be differentiable; with out= that raises, as torch's
    out= variants do."""
    import torch

    if _needs_grad(torch, x):
        if out is not None or handle_ is not None:
            raise RuntimeError("logsumexp(): out= and handle_ do not support automatic "
                               "differentiation, and x requires grad")
        return logsumexp_autograd(x)
    code, rows, cols, stride = _check_input(x)
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=x.device)
    elif out.dtype != torch.float32 or out.shape != (rows,) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor of shape (rows,)")
    dev, stream = _device_stream(x)
    h = handle_ if handle_ is not None else handle(dev, stream)
    lse_forward(h, x.data_ptr(), code, rows, cols, stride, out.data_ptr(), stream)
    return out


def token_logprob(x, targets, return_lse=False, handle_=None):
    """x[r, targets[r]] - LSE(x[r, :]) for a 2-D fp32/bf16/fp16 GPU tensor and an
    int64 GPU tensor of rows targets, as fp32[rows] (and the LSE, if asked).
    A target outside [0, cols) gives NaN. When x requires a gradient (and grad
    mode is on) this is token_logprob_autograd (which returns logp only, so
    return_lse=True raises there)."""
    import torch

    if _needs_grad(torch, x):
        if return_lse or handle_ is not None:
            raise RuntimeError("token_logprob(): return_lse=True and handle_ do not support "
                               "automatic differentiation; use token_logprob_autograd for the "
                               "gradient")
        return token_logprob_autograd(x, targets)
    code, rows, cols, stride = _check_input(x)
    if targets.dtype != torch.int64 or targets.shape != (rows,) or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int64 tensor of shape (rows,)")
    if targets.device != x.device:
        raise ValueError("targets must be on the same device as x")
    logp = torch.empty(rows, dtype=torch.float32, device=x.device)
    lse = torch.empty(rows, dtype=torch.float32, device=x.device) if return_lse else None
    dev, stream = _device_stream(x)
    h = handle_ if handle_ is not None else handle(dev, stream)
    lse_token_logprob(h, x.data_ptr(), code, rows, cols, stride, targets.data_ptr(),
                      logp.data_ptr(), lse.data_ptr() if lse is not None else None, stream)
    return (logp, lse) if return_lse else logp


def _autograd_function():
    import torch

    from .binding import lse_backward

    class _LogSumExp(torch.autograd.Function):
        """LSE over the last axis with the library's backward pass."""

        @staticmethod
        def forward(ctx, x):
            out = logsumexp(x)
            ctx.save_for_backward(x, out)
            return out

        @staticmethod
        def backward(ctx, grad_out):
            x, out = ctx.saved_tensors
            code, rows, cols, stride = _check_input(x)
            g = grad_out.to(torch.float32).contiguous()
            grad = torch.empty((rows, cols), dtype=x.dtype, device=x.device)
            dev, stream = _device_stream(x)
            h = handle(dev, stream)
            lse_backward(h, x.data_ptr(), code, rows, cols, stride, out.data_ptr(), g.data_ptr(),
                         grad.data_ptr(), cols, stream)
            return grad

    return _LogSumExp


_LSE_FN = None


def logsumexp_autograd(x):
    """LSE over the last axis of a 2-D fp32/bf16/fp16 GPU tensor, as fp32[rows],
    differentiable: the gradient with respect to x is grad_out[r] *
    exp(x[r, j] - lse[r]) (the row's softmax scaled by the incoming gradient),
    computed by the library's lse_backward and returned in x's dtype."""
    global _LSE_FN
    if _LSE_FN is None:
        _LSE_FN = _autograd_function()
    return _LSE_FN.apply(x)


def _token_autograd_function():
    import torch

    from .binding import lse_token_logprob, lse_token_logprob_backward

    class _TokenLogprob(torch.autograd.Function):
        """x[r, t[r]] - LSE(x[r, :]) with the library's backward pass."""

        @staticmethod
        def forward(ctx, x, targets):
            code, rows, cols, stride = _check_input(x)
            if targets.dtype != torch.int64 or targets.shape != (rows,) or \
                    not targets.is_contiguous() or targets.device != x.device:
                raise ValueError("targets must be a contiguous int64 tensor of shape (rows,) "
                                 "on x's device")
            logp = torch.empty(rows, dtype=torch.float32, device=x.device)
            lse = torch.empty(rows, dtype=torch.float32, device=x.device)
            dev, stream = _device_stream(x)
            h = handle(dev, stream)
            lse_token_logprob(h, x.data_ptr(), code, rows, cols, stride, targets.data_ptr(),
                              logp.data_ptr(), lse.data_ptr(), stream)
            ctx.save_for_backward(x, targets, lse)
            return logp

        @staticmethod
        def backward(ctx, grad_logp):
            x, targets, lse = ctx.saved_tensors
            code, rows, cols, stride = _check_input(x)
            g = grad_logp.to(torch.float32).contiguous()
            grad = torch.empty((rows, cols), dtype=x.dtype, device=x.device)
            dev, stream = _device_stream(x)
            h = handle(dev, stream)
            lse_token_logprob_backward(h, x.data_ptr(), code, rows, cols, stride,
                                       targets.data_ptr(), lse.data_ptr(), g.data_ptr(),
                                       grad.data_ptr(), cols, stream)
            return grad, None

    return _TokenLogprob


_TOK_FN = None


def token_logprob_autograd(x, targets):
    """x[r, targets[r]] - LSE(x[r, :]) for a 2-D fp32/bf16/fp16 GPU tensor, as
    fp32[rows], differentiable with respect to x: the gradient is
    grad_logp[r] * ([j == t] - exp(x[r, j] - lse[r])), computed by the
    library's lse_token_logprob_backward in x's dtype (NaN rows for targets
    outside [0, cols))."""
    global _TOK_FN
    if _TOK_FN is None:
        _TOK_FN = _token_autograd_function()
    return _TOK_FN.apply(x, targets)
