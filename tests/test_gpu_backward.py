"""GPU parity of the backward pass, lse_backward, against the float64 oracle:
grad_x[r, j] = grad_out[r] * exp(x[r, j] - lse[r]), with lse the forward value
as fp32 (here the oracle's LSE rounded to fp32, never the GPU's) and seeded
incoming gradients.

* Every workload's row prefix, every element compared.
* Every workload at full size: sampled rows element by element, and on every
  row the softmax sum: sum_j grad = g * exp(LSE - lse32).
* Ragged, padded and misaligned x and grad_x (vector and element paths), with
  special rows; nothing outside grad_x's rows is written.
"""
import numpy as np
import pytest

import workloads
from gpu_util import compare_grad, gpu_backward, note
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu

PREFIX = {1: 64, 2: 40, 3: 12, 4: 3000, 5: 300_000}
COLS = [1, 2, 3, 7, 8, 9, 16, 17, 33, 255, 257, 1023, 1024, 1025, 4097, 32001, 128257]


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


def decoded(x, dtype):
    return (workloads.bf16_bits_to_f32(x) if dtype == "bf16" else x).astype(np.float64)


def gap(x, dtype, lse32):
    """x - lse per element in float64 (NaN where both are infinite of one sign)."""
    with np.errstate(invalid="ignore"):
        return decoded(x, dtype) - lse32.astype(np.float64)[:, None]


def grads(rows, seed):
    rng = np.random.default_rng(seed)
    g = rng.normal(0, 2, size=rows).astype(np.float32)
    g[:: 7] = 1.0
    return g


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_prefix_all_elements(torch_gpu, handle, oracle, cfg):
    w = workloads.make(cfg, rows=PREFIX[cfg])
    lse32 = oracle.lse(w.x, w.dtype, threads=8).astype(np.float32)
    g = grads(w.rows, cfg)
    note(f"backward prefix cfg={cfg} rows={w.rows}")
    got, untouched = gpu_backward(torch_gpu, handle, w.x, lse32, g, w.dtype)
    assert untouched, "bytes outside grad_x's rows were written"
    ref = oracle.softmax_grad(w.x, lse32, g, w.dtype, threads=8)
    d = gap(w.x, w.dtype, lse32)
    compare_grad(got, ref, d, g, w.dtype, f"cfg{cfg} prefix")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size(torch_gpu, handle, oracle, cfg):
    w = workloads.make(cfg)
    lse = oracle.lse(w.x, w.dtype, threads=16)
    lse32 = lse.astype(np.float32)
    g = grads(w.rows, 10 + cfg)
    note(f"backward full cfg={cfg} shape={w.x.shape} dtype={w.dtype}")
    got, untouched = gpu_backward(torch_gpu, handle, w.x, lse32, g, w.dtype)
    assert untouched
    rng = np.random.default_rng(cfg)
    rows = np.unique(np.concatenate([rng.choice(w.rows, size=min(256, w.rows), replace=False),
                                     [0, w.rows - 1]]))
    sub = np.ascontiguousarray(w.x[rows])
    ref = oracle.softmax_grad(sub, lse32[rows], g[rows], w.dtype, threads=8)
    d = gap(sub, w.dtype, lse32[rows])
    compare_grad(got[rows], ref, d, g[rows], w.dtype, f"cfg{cfg} full sampled")
    # every row: the softmax sums to one, so sum_j grad = g * exp(LSE - lse32)
    fin = np.isfinite(lse)
    s = got[fin].sum(axis=1, dtype=np.float64)
    want = g[fin].astype(np.float64) * np.exp(lse[fin] - lse32[fin].astype(np.float64))
    rel = 2.0 ** -8 if w.dtype == "bf16" else 1e-5
    assert np.all(np.abs(s - want) <= rel * np.maximum(1.0, np.abs(want))), f"cfg{cfg} row sums"
    if cfg == 5:
        assert np.all(np.isnan(got[~fin])), "rows of only -inf: -inf - -inf"


def special_rows(dtype, rows, cols, seed):
    rng = np.random.default_rng(seed)
    v = rng.normal(0, 5, size=(rows, cols)).astype(np.float32)
    v[3 % rows] = -np.inf
    v[5 % rows, rng.integers(cols)] = np.nan
    v[7 % rows, rng.integers(cols)] = np.inf
    v[11 % rows] = 2.5
    v[13 % rows, : cols // 2] = -np.inf
    v[17 % rows] -= 200.0
    x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
    return x


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edges(torch_gpu, handle, oracle, dtype, cols):
    x = special_rows(dtype, 37, cols, seed=cols + len(dtype))
    lse32 = oracle.lse(x, dtype).astype(np.float32)
    g = grads(37, cols)
    ref = oracle.softmax_grad(x, lse32, g, dtype)
    d = gap(x, dtype, lse32)
    # (x front pad, grad row pad, grad front pad): aligned vectors, padded rows,
    # misaligned x (element path), misaligned grad (element path), both padded
    for front, gpad, gfront in [(0, 0, 0), (0, 5, 0), (1, 0, 0), (0, 0, 1), (0, 8, 8), (2, 3, 2)]:
        note(f"backward edges dtype={dtype} cols={cols} layout={(front, gpad, gfront)}")
        got, untouched = gpu_backward(torch_gpu, handle, x, lse32, g, dtype, pad_front=front,
                                      grad_pad=gpad, grad_front=gfront)
        assert untouched, f"writes outside grad rows {(front, gpad, gfront)}"
        compare_grad(got, ref, d, g, dtype, f"edges {dtype} cols={cols} {(front, gpad, gfront)}")


def test_padded_x_rows(torch_gpu, handle, oracle):
    """x with a row stride larger than cols (a view), vector and element paths."""
    rng = np.random.default_rng(9)
    for dtype in ["f32", "bf16"]:
        for cols, pad in [(1000, 24), (4096, 8), (17, 3), (100_000, 16)]:
            v = rng.normal(0, 3, size=(11, cols + pad)).astype(np.float32)
            full = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
            x = full[:, :cols]
            lse32 = oracle.lse(x, dtype).astype(np.float32)
            g = grads(11, cols)
            note(f"backward padded x dtype={dtype} cols={cols} pad={pad}")
            got, untouched = gpu_backward(torch_gpu, handle, x, lse32, g, dtype)
            assert untouched
            ref = oracle.softmax_grad(x, lse32, g, dtype)
            d = gap(np.ascontiguousarray(x), dtype, lse32)
            compare_grad(got, ref, d, g, dtype, f"padded x {dtype} cols={cols} pad={pad}")


def test_many_short_rows_block_boundaries(torch_gpu, handle, oracle):
    """Row counts around the rows-per-workgroup packing of short rows."""
    rng = np.random.default_rng(10)
    for dtype in ["f32", "bf16"]:
        for rows, cols in [(1, 16), (1023, 16), (1025, 16), (4097, 64), (70_001, 8), (3, 1000)]:
            v = rng.normal(0, 2, size=(rows, cols)).astype(np.float32)
            x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
            lse32 = oracle.lse(x, dtype).astype(np.float32)
            g = grads(rows, rows)
            note(f"backward rows={rows} cols={cols} dtype={dtype}")
            got, untouched = gpu_backward(torch_gpu, handle, x, lse32, g, dtype)
            assert untouched
            compare_grad(got, oracle.softmax_grad(x, lse32, g, dtype), gap(x, dtype, lse32), g, dtype,
                         f"rows={rows} cols={cols} {dtype}")


def test_empty_inputs(torch_gpu, handle):
    stream = torch_gpu.cuda.current_stream().cuda_stream
    B.lse_backward(handle, 0, B.LSE_DTYPE_F32, 0, 10, 10, 0, 0, 0, 10, stream)
    B.lse_backward(handle, 0, B.LSE_DTYPE_F32, 10, 0, 0, 0, 0, 0, 0, stream)
    torch_gpu.cuda.synchronize()


def test_forward_then_backward_matches_torch_autograd(torch_gpu, handle):
    """End to end on device memory: the library's forward, then its backward
    with that forward output, against torch.logsumexp's autograd in float64 on
    the CPU (a second, independent implementation of the same derivative)."""
    import row_wise_log_amd as R
    torch = torch_gpu
    rng = np.random.default_rng(11)
    v = rng.normal(0, 3, size=(50, 3000)).astype(np.float32)
    xg = torch.from_numpy(v).cuda()
    lse = R.logsumexp(xg)
    gout = torch.from_numpy(rng.normal(0, 1, size=50).astype(np.float32)).cuda()
    grad = torch.empty_like(xg)
    note("backward after forward")
    B.lse_backward(R.handle(0), xg.data_ptr(), B.LSE_DTYPE_F32, 50, 3000, 3000, lse.data_ptr(),
                   gout.data_ptr(), grad.data_ptr(), 3000, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    xc = torch.from_numpy(v).double().requires_grad_(True)
    torch.logsumexp(xc, dim=1).backward(gout.cpu().double())
    ref = xc.grad.numpy()
    got = grad.cpu().numpy().astype(np.float64)
    # the forward LSE is within 2e-6 * max(1, |LSE|) (|LSE| about 13 here), which
    # the backward carries as a relative error, plus its own 1e-6
    assert np.allclose(got, ref, rtol=3e-5, atol=1e-30), float(np.max(np.abs(got - ref)))


def test_package_autograd_against_torch(torch_gpu):
    """logsumexp_autograd: value and gradient (the library's lse_forward and
    lse_backward) against torch.logsumexp's float64 autograd on the CPU, for
    fp32 and bf16 inputs, contiguous and row-padded views."""
    import row_wise_log_amd as R
    torch = torch_gpu
    rng = np.random.default_rng(13)
    for dtype in (torch.float32, torch.bfloat16):
        for cols, pad in ((2049, 0), (1000, 24), (17, 3)):
            v = rng.normal(0, 3, size=(37, cols + pad)).astype(np.float32)
            big = torch.from_numpy(v).to("cuda", dtype).requires_grad_(True)
            x = big[:, :cols]
            note(f"package autograd dtype={dtype} cols={cols} pad={pad}")
            y = R.logsumexp_autograd(x)
            w = torch.from_numpy(rng.normal(0, 1, size=37).astype(np.float32)).cuda()
            (y * w).sum().backward()
            torch.cuda.synchronize()
            xc = x.detach().to(torch.float32).cpu().double().requires_grad_(True)
            yc = torch.logsumexp(xc, dim=1)
            (yc * w.cpu().double()).sum().backward()
            yv = y.detach().cpu().double().numpy()
            assert np.all(np.abs(yv - yc.detach().numpy()) <= 2e-6 * np.maximum(1, np.abs(yv)))
            assert big.grad.dtype == dtype
            g = big.grad.to(torch.float32).cpu().double().numpy()
            ref = xc.grad.numpy()
            # fp32: the forward's 2e-6 relative LSE error times |x - lse| (< 30 here)
            # plus the backward's own; bf16 output adds one rounding to 8 bits
            rel = 2.0 ** -8 + 1e-4 if dtype == torch.bfloat16 else 1e-4
            assert np.all(np.abs(g[:, :cols] - ref) <= rel * np.abs(ref) + 1e-30), (dtype, cols)
            assert np.all(g[:, cols:] == 0), "gradient leaked into the padding"
