"""GPU parity of the backward pass over a non-last axis, lse_backward_dim,
against the float64 oracle (oracle.lse_dim_grad: the row oracle's
softmax_grad over the moved axis):

    grad_x[o, j, i] = grad_out[o, i] * exp(x[o, j, i] - lse[o, i]),

with lse the oracle's LSE over j rounded to fp32 (never the GPU's) and seeded
incoming gradients. The bar is the row-wise backward pass's (compare_grad).

* Shapes [outer, n, inner] on the column tiles (16-bit types at widths that
  are multiples of the vector, rows on 128-byte lines or spanned by one tile)
  and the flat kernel (fp32, also with 4.8 MB of lse and grad_out; odd inner;
  16-bit rows off the 128-byte lines, inner 1032; a misaligned x, with grad_x at the same phase or not; fewer
  elements than one vector; n == 1 with several slices), fp32, bf16 and fp16;
  nothing outside grad_x is written.
* Forced splits of n (parts: the column tiles, both paths), special values
  (NaN, +-inf in x; infinite and NaN lse; zero and huge incoming gradients)
  on both kernels, inner == 1 (the row path).
* Workload 2 reduced over its first axis at full size, every element.
* The package's autograd wrapper over every axis of a 4-D tensor against
  torch.logsumexp's float64 autograd, and the plain helper's dispatch to it.
"""
import numpy as np
import pytest

import oracle as oracle_mod
import workloads
from gpu_util import gpu_dim_grad, note
from gpu_util import compare_dim_grad as check
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def handle(torch_gpu):
    h = B.lse_create(0)
    yield h
    torch_gpu.cuda.synchronize()
    B.lse_destroy(h)


def make(shape, dtype, seed, scale=3.0):
    v = np.random.default_rng(seed).normal(0, scale, size=shape).astype(np.float32)
    if dtype == "bf16":
        return workloads.f32_to_bf16_bits(v)
    if dtype == "f16":
        return workloads.f32_to_f16_bits(v)
    return v


def lse_and_grads(x3, dtype, seed):
    outer, _, inner = x3.shape
    lse2 = oracle_mod.lse_dim(x3, dtype, threads=8).astype(np.float32)
    g2 = np.random.default_rng(seed).normal(0, 2, size=(outer, inner)).astype(np.float32)
    return lse2, g2


SHAPES = [(1, 8192, 4096), (64, 1000, 32), (3, 5, 7), (2, 30_000, 3), (128, 17, 1024),
          (1, 1, 100), (7, 33, 12), (1, 3, 65), (16, 257, 40), (1, 64, 4 * 64 * 300),
          (2, 700, 1001), (1, 2, 3), (5, 1, 37), (3, 1000, 5001), (2, 300, 1032),
          (1, 4, 600_000)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_shapes(torch_gpu, handle, dtype, shape):
    x = make(shape, dtype, seed=sum(shape))
    lse2, g2 = lse_and_grads(x, dtype, seed=len(shape) + shape[1])
    # aligned; x misaligned (element path); grad_x misaligned alone (element path)
    for front, gfront in ((0, 0), (1, 1), (0, 1)):
        note(f"dim backward shape={shape} dtype={dtype} front={front} gfront={gfront}")
        got, untouched = gpu_dim_grad(torch_gpu, handle, x, lse2, g2, dtype, front, gfront)
        assert untouched, f"{shape} {dtype}: bytes outside grad_x were written"
        check(got, x, lse2, g2, dtype, f"dim backward {shape} {dtype} front={front},{gfront}")


@pytest.mark.parametrize("parts", [1, 3, 64])
def test_forced_parts(torch_gpu, handle, parts):
    """A forced `parts` selects the column tiles: their 16-byte path (inner
    256) and their one-column path (inner 257, which the planner otherwise
    gives to the flat kernel)."""
    for dtype in ["f32", "bf16"]:
        for inner in (256, 257):
            x = make((3, 5000, inner), dtype, seed=parts)
            lse2, g2 = lse_and_grads(x, dtype, seed=parts + 1)
            note(f"dim backward forced parts={parts} dtype={dtype} inner={inner}")
            got, untouched = gpu_dim_grad(torch_gpu, handle, x, lse2, g2, dtype, parts=parts)
            assert untouched
            check(got, x, lse2, g2, dtype, f"parts={parts} {dtype} inner={inner}")


def test_more_parts_than_rows(torch_gpu, handle):
    """Parts past the end of n are empty workgroups and write nothing."""
    x = make((2, 5, 512), "f32", seed=3)
    lse2, g2 = lse_and_grads(x, "f32", seed=4)
    note("dim backward parts > n")
    got, untouched = gpu_dim_grad(torch_gpu, handle, x, lse2, g2, "f32", parts=64)
    assert untouched
    check(got, x, lse2, g2, "f32", "parts > n")


@pytest.mark.parametrize("inner", [64, 63])
def test_special_values(torch_gpu, handle, inner):
    """Special values on the column tiles and the flat kernel (fp32, and any
    type at the odd width)."""
    rng = np.random.default_rng(9)
    for dtype in ["f32", "bf16"]:
        v = rng.normal(0, 2, size=(2, 300, inner)).astype(np.float32)
        v[0, :, 0] = -np.inf          # a column of only -inf (its LSE is -inf)
        v[0, 123, 1] = np.nan         # NaN
        v[0, 299, 2] = np.inf         # +inf (its LSE is +inf)
        v[1, :150, 4] = -np.inf       # half -inf
        v[1, 7, 5] = 80.0             # one large term
        x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
        lse2, g2 = lse_and_grads(x, dtype, seed=10)
        g2[0, 10] = 0.0               # a zero incoming gradient
        g2[1, 11] = 3.0e38            # a huge one
        lse2[1, 12] = np.nan          # a NaN lse
        lse2[1, 13] = np.inf          # an infinite lse with finite x: zero gradient
        for parts in (0, 1, 3):
            note(f"dim backward special values dtype={dtype} inner={inner} parts={parts}")
            got, untouched = gpu_dim_grad(torch_gpu, handle, x, lse2, g2, dtype, parts=parts)
            assert untouched
            check(got, x, lse2, g2, dtype, f"special {dtype} parts={parts}")


def test_inner_one_is_the_row_path(torch_gpu, handle):
    x = make((300, 777, 1), "bf16", seed=11)
    lse2, g2 = lse_and_grads(x, "bf16", seed=12)
    note("dim backward inner == 1")
    got, untouched = gpu_dim_grad(torch_gpu, handle, x, lse2, g2, "bf16")
    assert untouched
    check(got, x, lse2, g2, "bf16", "inner 1")


def test_empty(torch_gpu, handle):
    s = torch_gpu.cuda.current_stream().cuda_stream
    B.lse_backward_dim(handle, 0, B.LSE_DTYPE_F32, 3, 0, 9, 0, 0, 0, s)
    B.lse_backward_dim(handle, 0, B.LSE_DTYPE_F32, 0, 5, 9, 0, 0, 0, s)
    torch_gpu.cuda.synchronize()


def test_workload2_first_axis_full_size(torch_gpu, handle):
    """Workload 2 reduced over its first axis (outer 1, n 512, inner 128256):
    every element of the gradient against the oracle."""
    w = workloads.make(2)
    x3 = w.x.reshape(1, w.rows, w.cols)
    lse2, g2 = lse_and_grads(x3, "bf16", seed=20)
    note("dim backward workload 2 over axis 0")
    got, untouched = gpu_dim_grad(torch_gpu, handle, x3, lse2, g2, "bf16")
    assert untouched
    check(got, x3, lse2, g2, "bf16", "workload 2 axis 0")


def test_short_rows_in_one_batch_parts(torch_gpu, handle):
    """Rows of 16 fp32 over a long axis (a tile spans whole rows, so n is cut
    into parts of one batch per lane, up to 65536 of them): 2^20 rows, every
    element against the oracle."""
    x = make((1, 1 << 20, 16), "f32", seed=22)
    lse2, g2 = lse_and_grads(x, "f32", seed=23)
    note("dim backward 2^20 rows of 16 fp32")
    got, untouched = gpu_dim_grad(torch_gpu, handle, x, lse2, g2, "f32")
    assert untouched
    check(got, x, lse2, g2, "f32", "rows of 16")


def test_package_autograd_every_axis(torch_gpu):
    """logsumexp_dim_autograd, and logsumexp_dim on a tensor that requires a
    gradient, against torch.logsumexp's float64 autograd on the CPU for every
    axis of a 4-D tensor (fp32 and bf16), keepdim both ways."""
    import row_wise_log_amd as R
    torch = torch_gpu
    rng = np.random.default_rng(21)
    v = rng.normal(0, 3, size=(3, 40, 7, 9)).astype(np.float32)
    for dtype in (torch.float32, torch.bfloat16):
        for dim in range(4):
            for keepdim in (False, True):
                for fn in (R.logsumexp_dim_autograd, R.logsumexp_dim):
                    note(f"dim autograd dtype={dtype} dim={dim} keepdim={keepdim} {fn.__name__}")
                    x = torch.from_numpy(v).to("cuda", dtype).requires_grad_(True)
                    y = fn(x, dim, keepdim)
                    assert y.grad_fn is not None
                    w = torch.from_numpy(rng.normal(0, 1, size=tuple(y.shape)).astype(np.float32))
                    (y * w.cuda()).sum().backward()
                    torch.cuda.synchronize()
                    xc = x.detach().to(torch.float32).cpu().double().requires_grad_(True)
                    yc = torch.logsumexp(xc, dim=dim, keepdim=keepdim)
                    (yc * w.double()).sum().backward()
                    yv = y.detach().cpu().double().numpy()
                    assert np.all(np.abs(yv - yc.detach().numpy()) <= 1e-5 * np.maximum(1, np.abs(yv)))
                    assert x.grad.dtype == dtype and x.grad.shape == x.shape
                    g = x.grad.to(torch.float32).cpu().double().numpy()
                    ref = xc.grad.numpy()
                    rel = 2.0 ** -8 + 1e-4 if dtype == torch.bfloat16 else 1e-4
                    assert np.all(np.abs(g - ref) <= rel * np.abs(ref) + 1e-30), (dtype, dim)
