"""Byte offsets beyond 2^31 and 2^32: rows 4 GiB apart, and a non-last-axis
reduction over arrays of 6 to 9 GB (an MI355X holds 288 GB).

* lse_forward, lse_token_logprob and lse_backward on 3 rows placed 2^30 + 64
  fp32 elements (4 GiB + 256 bytes) or 2^31 + 64 bf16 elements apart, for a
  register-rows width and a streaming width; results against the oracle, and
  the backward's output buffer (filled with a pattern no gradient can take)
  changes in exactly rows x cols elements.
* lse_forward_dim over [1, n, inner] with inner = 2^30 + 8 (bf16, vector
  path) and 2^29 + 3 (fp32, element path): all columns zero except 64
  sampled ones, so every untouched output must be ln n; the sampled columns
  against the oracle.
* lse_backward_dim over [1, 65536, 40000] bf16 (5.2 GB, column tiles) and
  [1, 40000, 40001] fp32 (6.4 GB, the flat kernel): every gradient of the
  zero columns must be the same constant g / n; the sampled columns against
  the oracle; nothing written past grad_x.
"""
import math

import numpy as np
import pytest

import oracle as oracle_mod
import workloads
from gpu_util import DTYPE_CODE, compare, compare_grad, compare_logp, note
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


def _rows(dtype, rows, cols, seed):
    v = np.random.default_rng(seed).normal(0, 4, size=(rows, cols)).astype(np.float32)
    v[1, cols // 3] = 40.0
    return workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v


@pytest.mark.parametrize("dtype,stride", [("f32", (1 << 30) + 64), ("bf16", (1 << 31) + 64)])
@pytest.mark.parametrize("cols", [1000, 300_000])
def test_rows_four_gib_apart(torch_gpu, handle, oracle, dtype, stride, cols):
    torch = torch_gpu
    rows = 3
    st = torch.int16 if dtype == "bf16" else torch.int32
    host = _rows(dtype, rows, cols, seed=cols)
    hv = host.view(np.int16 if dtype == "bf16" else np.int32)
    n = (rows - 1) * stride + cols
    note(f"large offsets {dtype} stride={stride} cols={cols}: {n * host.itemsize / 2**30:.1f} GiB")
    x = torch.zeros(n, dtype=st, device="cuda")
    for r in range(rows):
        x[r * stride: r * stride + cols] = torch.from_numpy(hv[r].copy()).cuda()
    code, s = DTYPE_CODE[dtype], torch.cuda.current_stream().cuda_stream
    ref = oracle.lse(host, dtype)
    out = torch.full((rows,), float("nan"), device="cuda")
    B.lse_forward(handle, x.data_ptr(), code, rows, cols, stride, out.data_ptr(), s)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), ref, dtype, f"forward {dtype} cols={cols}")
    targets = np.array([0, cols // 3, cols - 1], dtype=np.int64)
    logp = torch.empty(rows, device="cuda")
    tg = torch.from_numpy(targets).cuda()   # kept alive until the call has run
    B.lse_token_logprob(handle, x.data_ptr(), code, rows, cols, stride, tg.data_ptr(),
                        logp.data_ptr(), None, s)
    torch.cuda.synchronize()
    compare_logp(logp.cpu().numpy(), oracle.token_logprob(host, targets, dtype), ref, dtype,
                 f"token logprob {dtype} cols={cols}")
    # backward into an equally spread gradient buffer, pre-filled with a pattern
    # (bf16 0x7F7F, fp32 0x7F7F7F7F: about 3.4e38) that no gradient here can take
    lse32 = ref.astype(np.float32)
    g = np.array([1.0, -2.0, 0.5], dtype=np.float32)
    sentinel = 0x7F7F if dtype == "bf16" else 0x7F7F7F7F
    gx = torch.full((n,), sentinel, dtype=st, device="cuda")
    # the device copies of lse and g must outlive the call: a temporary freed
    # while the arguments are evaluated would hand its memory to the next one
    lt, gt = torch.from_numpy(lse32).cuda(), torch.from_numpy(g).cuda()
    B.lse_backward(handle, x.data_ptr(), code, rows, cols, stride, lt.data_ptr(), gt.data_ptr(),
                   gx.data_ptr(), stride, s)
    torch.cuda.synchronize()
    assert int((gx != sentinel).sum()) == rows * cols, "writes outside grad_x's rows"
    got = np.stack([gx[r * stride: r * stride + cols].cpu().numpy() for r in range(rows)])
    got = (workloads.bf16_bits_to_f32(got.view(np.uint16)) if dtype == "bf16"
           else got.view(np.float32))
    vals = (workloads.bf16_bits_to_f32(host) if dtype == "bf16" else host).astype(np.float64)
    compare_grad(got, oracle.softmax_grad(host, lse32, g, dtype),
                 vals - lse32.astype(np.float64)[:, None], g, dtype, f"backward {dtype} cols={cols}")
    del x, gx, lt, gt, tg


@pytest.mark.parametrize("dtype,n,inner", [("bf16", 3, (1 << 30) + 8), ("f32", 4, (1 << 29) + 3)])
def test_dim_over_large_arrays(torch_gpu, handle, dtype, n, inner):
    torch = torch_gpu
    st = torch.int16 if dtype == "bf16" else torch.int32
    note(f"large dim {dtype} n={n} inner={inner}: {n * inner * (2 if dtype == 'bf16' else 4) / 1e9:.1f} GB")
    x = torch.zeros((n, inner), dtype=st, device="cuda")
    rng = np.random.default_rng(inner)
    cols = np.unique(np.concatenate([rng.integers(0, inner, size=60), [0, 1, inner - 2, inner - 1]]))
    vals = rng.normal(0, 5, size=(n, len(cols))).astype(np.float32)
    vals[0, 0] = 60.0
    hv = workloads.f32_to_bf16_bits(vals) if dtype == "bf16" else vals
    idx = torch.from_numpy(cols).cuda()
    x[:, idx] = torch.from_numpy(hv.view(np.int16 if dtype == "bf16" else np.int32)).cuda()
    out = torch.full((inner,), float("nan"), device="cuda")
    B.lse_forward_dim(handle, x.data_ptr(), DTYPE_CODE[dtype], 1, n, inner, out.data_ptr(),
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ln_n = math.log(n)
    mask = torch.ones(inner, dtype=torch.bool, device="cuda")
    mask[idx] = False
    tol = 1e-5 if dtype == "bf16" else 2e-6
    bad = int(((out - ln_n).abs() > tol * max(1.0, ln_n))[mask].sum())
    assert bad == 0, f"{bad} untouched columns differ from ln {n}"
    ref = oracle_mod.lse(np.ascontiguousarray(hv.T), dtype)   # each sampled column is a row of n
    compare(out[idx].cpu().numpy(), ref, dtype, f"dim {dtype} sampled columns")
    del x, out


@pytest.mark.parametrize("dtype,n,inner", [("bf16", 65536, 40000), ("f32", 40000, 40001)])
def test_dim_backward_over_a_large_array(torch_gpu, handle, dtype, n, inner):
    """lse_backward_dim over [1, 65536, 40000] bf16 (2.6 G elements, 5.2 GB;
    the column tiles' 16-byte path) and [1, 40000, 40001] fp32 (1.6 G
    elements, 6.4 GB; the flat kernel), byte offsets past 2^32: x = 0 except a
    few sampled columns, so every other column's gradient is exactly g / n
    for g = 1 and lse = fl(ln n) (2^-16 for n = 65536; for n = 40000 the
    constant the same formula gives in fp32, computed on the host); the
    sampled columns are checked against the oracle, and the guard after
    grad_x stays untouched."""
    torch = torch_gpu
    esize = 2 if dtype == "bf16" else 4
    st = torch.int16 if dtype == "bf16" else torch.int32
    note(f"large dim backward {dtype} n={n} inner={inner}: {n * inner * esize / 1e9:.1f} GB")
    x = torch.zeros((n, inner), dtype=st, device="cuda")
    rng = np.random.default_rng(7)
    cols = np.unique(np.concatenate([rng.integers(0, inner, size=20), [0, inner - 1]]))
    vals = rng.normal(0, 3, size=(n, len(cols))).astype(np.float32)
    hv = workloads.f32_to_bf16_bits(vals) if dtype == "bf16" else vals
    idx = torch.from_numpy(cols).cuda()
    x[:, idx] = torch.from_numpy(hv.view(np.int16 if dtype == "bf16" else np.int32)).cuda()
    lse = np.full(inner, math.log(n), dtype=np.float32)
    lse[cols] = oracle_mod.lse(np.ascontiguousarray(hv.T), dtype).astype(np.float32)
    g = np.ones(inner, dtype=np.float32)
    g[cols] = rng.normal(0, 2, size=len(cols)).astype(np.float32)
    lt, gt = torch.from_numpy(lse).cuda(), torch.from_numpy(g).cuda()
    guard = 16384 // esize
    sentinel = 0x7F7F if dtype == "bf16" else 0x7F7F7F7F
    grad = torch.full((n * inner + guard,), sentinel, dtype=st, device="cuda")
    B.lse_backward_dim(handle, x.data_ptr(), DTYPE_CODE[dtype], 1, n, inner, lt.data_ptr(),
                       gt.data_ptr(), grad.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert bool((grad[n * inner:] == sentinel).all()), "the guard after grad_x was written"
    gv = grad[: n * inner].view(n, inner)
    mask = torch.ones(inner, dtype=torch.bool, device="cuda")
    mask[idx] = False
    # the zero columns' gradient: 1 * 2^((0 - fl(ln n)) * fl(log2 e)) in fp32,
    # which is exactly 2^-16 for n = 65536; compared as the stored bits
    c = np.float32(np.float32(0.0) - np.float32(math.log(n))) * np.float32(math.log2(math.e))
    want = np.array([np.exp2(np.float64(c))], dtype=np.float32)
    if n == 65536:
        assert want[0] == np.float32(2.0 ** -16)
    if dtype == "bf16":
        want_bits = int(workloads.f32_to_bf16_bits(want)[0])
        bad = int((gv[:, mask] != want_bits).sum())
        assert bad == 0, f"{bad} elements of the constant columns differ from g / n"
    else:
        # v_exp_f32 is within 1 ulp of 2^c: the constant columns agree with it
        # to that and with each other exactly
        const = gv[:, mask].view(torch.float32)
        first = const[0, 0].item()
        assert abs(first - float(want[0])) <= 2.0 ** -23 * float(want[0]) * 2
        assert bool((const == first).all()), "the constant columns differ from each other"
    got = gv[:, idx].cpu().numpy()
    if dtype == "bf16":
        got = (got.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    else:
        got = got.view(np.float32)
    got = got.astype(np.float64)
    ref = oracle_mod.softmax_grad(np.ascontiguousarray(hv.T), lse[cols], g[cols], dtype).T
    rel = 2.0 ** -8 + 1e-6 if dtype == "bf16" else 4e-7  # as compare_grad
    xv = workloads.bf16_bits_to_f32(hv) if dtype == "bf16" else hv
    d = np.abs(xv.astype(np.float64) - lse[cols][None, :])
    tol = (rel + 2e-7 * d) * np.abs(ref) + 2.0 ** -125 * np.maximum(1.0, np.abs(g[cols]))[None, :]
    assert np.all(np.abs(got - ref) <= tol), "sampled columns differ from the oracle"
    del x, grad, gv
