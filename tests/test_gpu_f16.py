"""GPU parity for IEEE half (fp16) inputs, through every entry point.

The 16-bit reading of the paper's reduced-bit FuseLSE16 (§4.3, Figure 5):
the same single pass over 16-bit data, decoded exactly and accumulated in
fp32, so the forward bar is bf16's (1e-5 * max(1, |LSE|)) against the
oracle on the same fp16 bits. Covered: the headline shape's values stored
as fp16 (prefix under every schedule, full size on every row), the many
short rows of workload 5 (register rows, deferred stores), widths around
every vector and tail boundary in contiguous, padded and misaligned
layouts with special rows, the half format's own extremes (65504, the
smallest subnormal, overflow to +inf), the token log-probability, both
backward passes (fp16 gradients rounded once from fp32), the non-last-axis
LSE, the no-allocation entry point and the torch helpers on float16
tensors against torch's float64 results.
"""
import numpy as np
import pytest

import workloads
from gpu_util import (SCHEDULES, compare, compare_grad, compare_logp, compare_token_grad,
                      gpu_backward, gpu_lse, gpu_token_backward, gpu_token_logprob, note, upload)
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu

F16 = "f16"


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


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def make_rows(rows, cols, layout, seed, scale=5.0):
    """fp16 bits of random rows with special rows mixed in (as the bf16 / fp32
    edge tests); returns (array view, pad_front)."""
    rng = np.random.default_rng(seed)
    pad = {"contiguous": 0, "padded": 5, "misaligned": 0}[layout]
    v = rng.normal(0, scale, size=(rows, cols + pad)).astype(np.float32)
    if cols:
        v[3 % rows] = -np.inf
        v[5 % rows, rng.integers(cols)] = np.nan
        v[7 % rows, rng.integers(cols)] = np.inf
        v[11 % rows] = 2.5
        v[13 % rows, : cols // 2] = -np.inf
        v[17 % rows] -= 200.0
        v[19 % rows, rng.integers(cols)] = 60000.0     # near the top of the half range
        v[23 % rows] = 2.0 ** -20                       # subnormal halves
    x = workloads.f32_to_f16_bits(v)
    x = x[:, :cols] if pad else x
    return x, (1 if layout == "misaligned" else 0)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_headline_values_as_f16_every_schedule(torch_gpu, handle, oracle, schedule):
    w = workloads.make(2, rows=40, storage=F16)
    note(f"f16 headline prefix schedule={schedule}")
    got = gpu_lse(torch_gpu, handle, w.x, F16, schedule)
    compare(got, oracle.lse(w.x, F16, threads=8), F16, f"f16 headline prefix {schedule}")


def test_headline_values_as_f16_full_size(torch_gpu, handle, oracle):
    w = workloads.make(2, storage=F16)
    note("f16 headline full size")
    got = gpu_lse(torch_gpu, handle, w.x, F16, "auto")
    compare(got, oracle.lse(w.x, F16, threads=16), F16, "f16 headline full, every row")


@pytest.mark.parametrize("schedule", ["auto", "rows_per_wave", "row_per_wg"])
def test_short_rows_as_f16(torch_gpu, handle, oracle, schedule):
    """Workload 5's rows of 16 (log-probabilities, -inf entries and rows)
    stored as fp16: the register-rows plan with its deferred stores."""
    w = workloads.make(5, rows=300_000, storage=F16)
    note(f"f16 short rows schedule={schedule}")
    got = gpu_lse(torch_gpu, handle, w.x, F16, schedule)
    compare(got, oracle.lse(w.x, F16, threads=8), F16, f"f16 short rows {schedule}")


COLS = [0, 1, 7, 8, 9, 15, 16, 17, 63, 64, 65, 511, 1024, 1025, 4095, 4096, 4097, 20001,
        65536, 128257]


@pytest.mark.parametrize("layout", ["contiguous", "padded", "misaligned"])
@pytest.mark.parametrize("cols", COLS)
def test_edge_sweep_f16(torch_gpu, handle, oracle, cols, layout):
    x, front = make_rows(37, cols, layout, seed=cols * 11 + len(layout))
    ref = oracle.lse(x, F16)
    for sched in SCHEDULES:
        note(f"f16 edge cols={cols} layout={layout} schedule={sched}")
        got = gpu_lse(torch_gpu, handle, x, F16, sched, pad_front=front)
        compare(got, ref, F16, f"f16 cols={cols} {layout} {sched}")


def test_half_range_extremes(torch_gpu, handle, oracle):
    """Rows at the top of the half range (65504, whose sum exceeds the half
    range but not fp32's), of the smallest subnormal, and of +-inf / NaN."""
    rows = [np.full(1000, 0x7BFF), np.full(1000, 0x0001), np.full(1000, 0x8001),
            np.array([0x7BFF] * 500 + [0xFC00] * 500), np.array([0x7C00] + [0x3C00] * 999),
            np.array([0x7E00] + [0x3C00] * 999), np.full(1000, 0xFC00)]
    x = np.stack(rows).astype(np.uint16)
    ref = oracle.lse(x, F16)
    assert ref[0] == pytest.approx(65504.0 + np.log(1000.0), rel=1e-15)
    for sched in SCHEDULES:
        note(f"f16 extremes schedule={sched}")
        compare(gpu_lse(torch_gpu, handle, x, F16, sched), ref, F16, f"f16 extremes {sched}")


@pytest.mark.parametrize("cols", [5, 16, 1000, 128256])
def test_token_logprob_f16(torch_gpu, handle, oracle, cols):
    x, _ = make_rows(64, cols, "contiguous", seed=cols)
    rng = np.random.default_rng(cols + 1)
    t = rng.integers(0, cols, size=64)
    t[:3] = [0, cols - 1, cols]  # both ends, and one out of range
    ref_lse = oracle.lse(x, F16)
    ref = oracle.token_logprob(x, t, F16)
    for sched in SCHEDULES:
        note(f"f16 token logprob cols={cols} schedule={sched}")
        logp, lse = gpu_token_logprob(torch_gpu, handle, x, t, F16, sched)
        compare(lse, ref_lse, F16, f"f16 token lse cols={cols} {sched}")
        compare_logp(logp, ref, ref_lse, F16, f"f16 logp cols={cols} {sched}")


@pytest.mark.parametrize("layout", [(0, 0, 0), (1, 3, 1)])
@pytest.mark.parametrize("cols", [1, 9, 1024, 50257])
def test_backward_f16(torch_gpu, handle, oracle, cols, layout):
    """grad_out * exp(x - lse) written as fp16 (one rounding from fp32), in
    aligned and misaligned / padded layouts; nothing outside the rows written."""
    pad_front, grad_pad, grad_front = layout
    x, _ = make_rows(24, cols, "contiguous", seed=cols + 7, scale=3.0)
    lse32 = oracle.lse(x, F16).astype(np.float32)
    g = np.random.default_rng(cols).normal(0, 1, size=24).astype(np.float32)
    note(f"f16 backward cols={cols} layout={layout}")
    got, untouched = gpu_backward(torch_gpu, handle, x, lse32, g, F16, pad_front, grad_pad,
                                  grad_front)
    assert untouched
    ref = oracle.softmax_grad(x, lse32, g, F16)
    with np.errstate(invalid="ignore"):
        d = f16_values(x) - lse32.astype(np.float64)[:, None]
    compare_grad(got, ref, d, g, F16, f"f16 backward cols={cols} {layout}")
    t = np.random.default_rng(cols + 3).integers(0, cols, size=24)
    note(f"f16 token backward cols={cols} layout={layout}")
    got, untouched = gpu_token_backward(torch_gpu, handle, x, t, lse32, g, F16, pad_front,
                                        grad_pad, grad_front)
    assert untouched
    ref = oracle.token_logprob_grad(x, t, lse32, g, F16)
    compare_token_grad(got, ref, oracle.softmax_grad(x, lse32, g, F16), d, g, t, F16,
                       f"f16 token backward cols={cols} {layout}")


@pytest.mark.parametrize("shape,front", [((1, 8192, 4096), 0), ((64, 1000, 32), 0),
                                         ((3, 5, 7), 0), ((16, 257, 40), 1), ((2, 100_000, 3), 0),
                                         ((1, 4096, 4097), 0), ((1, 20_000, 1025), 1),
                                         ((1, 1_000_000, 8), 0)])
def test_dim_f16(torch_gpu, handle, shape, front):
    """lse_forward_dim on fp16: the 16-byte path, the one-column path unsplit
    and split (16-step batches, about two workgroups per CU), a misaligned
    base, and one column group per row (lanes sharing columns in the end
    merge)."""
    import oracle as orc
    torch = torch_gpu
    v = np.random.default_rng(sum(shape)).normal(0, 4, size=shape).astype(np.float32)
    x3 = workloads.f32_to_f16_bits(v)
    outer, n, inner = shape
    flat = np.zeros(front + x3.size, dtype=np.uint16)
    flat[front:] = x3.ravel()
    t = torch.from_numpy(flat.view(np.int16)).to("cuda")
    out = torch.full((outer * inner,), 123.0, dtype=torch.float32, device="cuda")
    note(f"f16 dim shape={shape} front={front}")
    B.lse_forward_dim(handle, t.data_ptr() + 2 * front, B.LSE_DTYPE_F16, outer, n, inner,
                      out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = orc.lse_dim(x3, F16).ravel()
    compare(out.cpu().numpy(), ref, F16, f"f16 dim {shape}")


def test_noalloc_f16(torch_gpu, handle, oracle):
    torch = torch_gpu
    w = workloads.make(2, rows=24, storage=F16)
    t, ptr, stride = upload(torch, w.x)
    out = torch.empty(24, device="cuda")
    note("f16 noalloc")
    B.lse_forward_noalloc(ptr, B.LSE_DTYPE_F16, 24, w.cols, stride, out.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), gpu_lse(torch, handle, w.x, F16).view(np.uint32))
    compare(got, oracle.lse(w.x, F16), F16, "f16 noalloc")


def test_package_helpers_on_float16(torch_gpu):
    """logsumexp, logsumexp_dim and logsumexp_autograd on float16 tensors
    against torch's float64 results on the same values."""
    import row_wise_log_amd as lib
    torch = torch_gpu
    g = torch.Generator(device="cpu").manual_seed(9)
    x = (torch.randn(300, 5000, generator=g) * 4).to(torch.float16).cuda()
    note("f16 package helpers")
    ref = torch.logsumexp(x.double(), dim=1)
    got = lib.logsumexp(x)
    assert torch.allclose(got.double(), ref, rtol=1e-5, atol=1e-5)
    x4 = (torch.randn(3, 40, 7, 9, generator=g) * 3).to(torch.float16).cuda()
    for d in range(4):
        ref = torch.logsumexp(x4.double(), dim=d)
        assert torch.allclose(lib.logsumexp_dim(x4, d).double(), ref, rtol=1e-5, atol=1e-5), d
    xr = x[:37].clone().requires_grad_(True)
    lib.logsumexp_autograd(xr).sum().backward()
    x64 = x[:37].double().clone().requires_grad_(True)
    torch.logsumexp(x64, dim=1).sum().backward()
    assert xr.grad.dtype == torch.float16
    # the forward's LSE error (1e-5 of max(1, |LSE|), |LSE| < 40 here) carried
    # into exp(x - lse), and one fp16 rounding: 2^-11 relative, 2^-25 absolute
    err = (xr.grad.double() - x64.grad).abs()
    assert bool((err <= (2.0 ** -11 + 4e-4) * x64.grad.abs() + 2.0 ** -25).all())
