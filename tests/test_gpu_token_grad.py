"""GPU parity of the token log-probability's backward pass,
lse_token_logprob_backward, against the float64 oracle:
grad_x[r, j] = g[r] * ([j == t_r] - exp(x[r, j] - lse[r])), with lse the
oracle's LSE rounded to fp32 (never the GPU's) and seeded targets and
incoming gradients.

* Every workload's row prefix, every element compared; each workload at full
  size with sampled rows compared element by element and, on every row, the
  row sum g * (1 - exp(LSE - lse32)).
* Widths from 1 to 128257 in fp32 and bf16, with padded and misaligned x and
  grad_x (vector and element paths), targets at both ends, in the vector tail
  and out of range (rows of NaN), and special rows; nothing outside grad_x's
  rows is written.
* Row counts around the packing of short rows, and the package's
  token_logprob_autograd against torch's log_softmax + gather autograd.
"""
import numpy as np
import pytest

import workloads
from gpu_util import compare_token_grad, gpu_token_backward, note
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu

PREFIX = {1: 64, 2: 40, 3: 12, 4: 3000, 5: 300_000}
COLS = [1, 2, 3, 7, 8, 9, 16, 17, 33, 255, 257, 1024, 1025, 4097, 32001, 128257]


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


def gap(x, dtype, lse32):
    vals = (workloads.bf16_bits_to_f32(x) if dtype == "bf16" else x).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return vals - lse32.astype(np.float64)[:, None]


def grads(rows, seed):
    g = np.random.default_rng(seed).normal(0, 2, size=rows).astype(np.float32)
    g[::5] = 1.0
    return g


def check(oracle, got, x, targets, lse32, g, dtype, what):
    xc = np.ascontiguousarray(x)
    ref = oracle.token_logprob_grad(xc, targets, lse32, g, dtype, threads=8)
    soft = oracle.softmax_grad(xc, lse32, g, dtype, threads=8)
    compare_token_grad(got, ref, soft, gap(xc, dtype, lse32), g, targets, dtype, what)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_prefix_all_elements(torch_gpu, handle, oracle, cfg):
    w = workloads.make(cfg, rows=PREFIX[cfg])
    t = workloads.targets(cfg, w.rows)
    lse32 = oracle.lse(w.x, w.dtype, threads=8).astype(np.float32)
    g = grads(w.rows, cfg)
    note(f"token backward prefix cfg={cfg} rows={w.rows}")
    got, untouched = gpu_token_backward(torch_gpu, handle, w.x, t, lse32, g, w.dtype)
    assert untouched, "bytes outside grad_x's rows were written"
    check(oracle, got, w.x, t, lse32, g, w.dtype, f"cfg{cfg} prefix")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size(torch_gpu, handle, oracle, cfg):
    w = workloads.make(cfg)
    t = workloads.targets(cfg)
    lse = oracle.lse(w.x, w.dtype, threads=16)
    lse32 = lse.astype(np.float32)
    g = grads(w.rows, 20 + cfg)
    note(f"token backward full cfg={cfg} shape={w.x.shape}")
    got, untouched = gpu_token_backward(torch_gpu, handle, w.x, t, lse32, g, w.dtype)
    assert untouched
    rng = np.random.default_rng(cfg)
    rows = np.unique(np.concatenate([rng.choice(w.rows, size=min(256, w.rows), replace=False),
                                     [0, w.rows - 1]]))
    check(oracle, got[rows], np.ascontiguousarray(w.x[rows]), t[rows], lse32[rows], g[rows],
          w.dtype, f"cfg{cfg} full sampled")
    # every row: the one-hot term and the softmax each sum to one
    fin = np.isfinite(lse)
    s = got[fin].sum(axis=1, dtype=np.float64)
    want = g[fin].astype(np.float64) * (1.0 - np.exp(lse[fin] - lse32[fin].astype(np.float64)))
    bar = (2.0 ** -6 if w.dtype == "bf16" else 1e-5) * np.maximum(1.0, np.abs(g[fin]))
    assert np.all(np.abs(s - want) <= bar), f"cfg{cfg} row sums"


def special_rows(dtype, rows, cols, seed):
    rng = np.random.default_rng(seed)
    v = rng.normal(0, 5, size=(rows, cols)).astype(np.float32)
    v[3 % rows] = -np.inf
    v[5 % rows, rng.integers(cols)] = np.nan
    v[7 % rows, rng.integers(cols)] = np.inf
    v[11 % rows] = 2.5
    v[13 % rows, : cols // 2] = -np.inf
    v[17 % rows] -= 200.0
    return workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v


def edge_targets(rows, cols, seed):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, cols, size=rows)
    t[0], t[1 % rows], t[2 % rows] = 0, cols - 1, -1
    t[4 % rows] = cols                       # just past the end: NaN row
    t[6 % rows] = (cols // 8) * 8 if cols >= 8 else cols - 1   # first element of the vector tail
    t[8 % rows] = 1 << 40
    return t


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edges(torch_gpu, handle, oracle, dtype, cols):
    x = special_rows(dtype, 37, cols, seed=cols + len(dtype))
    t = edge_targets(37, cols, cols)
    lse32 = oracle.lse(x, dtype).astype(np.float32)
    g = grads(37, cols)
    for front, gpad, gfront in [(0, 0, 0), (0, 5, 0), (1, 0, 0), (0, 0, 1), (2, 3, 2)]:
        note(f"token backward edges dtype={dtype} cols={cols} layout={(front, gpad, gfront)}")
        got, untouched = gpu_token_backward(torch_gpu, handle, x, t, lse32, g, dtype, pad_front=front,
                                            grad_pad=gpad, grad_front=gfront)
        assert untouched, f"writes outside grad rows {(front, gpad, gfront)}"
        check(oracle, got, x, t, lse32, g, dtype, f"edges {dtype} cols={cols} {(front, gpad, gfront)}")


def test_many_short_rows(torch_gpu, handle, oracle):
    """Row counts around the packing of short rows (several rows per workgroup)."""
    rng = np.random.default_rng(40)
    for dtype in ["f32", "bf16"]:
        for rows, cols in [(1, 16), (1023, 16), (1025, 16), (4097, 64), (70_001, 8), (3, 1000)]:
            v = rng.normal(0, 2, size=(rows, cols)).astype(np.float32)
            x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
            t = rng.integers(0, cols, size=rows)
            lse32 = oracle.lse(x, dtype).astype(np.float32)
            g = grads(rows, rows)
            note(f"token backward rows={rows} cols={cols} dtype={dtype}")
            got, untouched = gpu_token_backward(torch_gpu, handle, x, t, lse32, g, dtype)
            assert untouched
            check(oracle, got, x, t, lse32, g, dtype, f"rows={rows} cols={cols} {dtype}")


def test_package_autograd_against_torch(torch_gpu):
    """token_logprob_autograd: value and gradient (the library's fused forward
    and lse_token_logprob_backward) against log_softmax + gather in float64 on
    the CPU, fp32 and bf16, contiguous and row-padded views."""
    import row_wise_log_amd as R
    torch = torch_gpu
    rng = np.random.default_rng(41)
    for dtype in (torch.float32, torch.bfloat16):
        for cols, pad in ((2049, 0), (1000, 24), (17, 3)):
            v = rng.normal(0, 3, size=(29, cols + pad)).astype(np.float32)
            big = torch.from_numpy(v).to("cuda", dtype).requires_grad_(True)
            x = big[:, :cols]
            t = torch.from_numpy(rng.integers(0, cols, size=29)).cuda()
            note(f"package token autograd dtype={dtype} cols={cols} pad={pad}")
            logp = R.token_logprob_autograd(x, t)
            w = torch.from_numpy(rng.normal(0, 1, size=29).astype(np.float32)).cuda()
            (logp * w).sum().backward()
            torch.cuda.synchronize()
            xc = x.detach().to(torch.float32).cpu().double().requires_grad_(True)
            ref = torch.log_softmax(xc, dim=1).gather(1, t.cpu()[:, None])[:, 0]
            (ref * w.cpu().double()).sum().backward()
            lv = logp.detach().cpu().double().numpy()
            assert np.all(np.abs(lv - ref.detach().numpy()) <= 2e-5 * np.maximum(1, np.abs(lv)))
            assert big.grad.dtype == dtype
            got = big.grad.to(torch.float32).cpu().double().numpy()[:, :cols]
            want = xc.grad.numpy()
            scale = np.abs(w.cpu().double().numpy())[:, None]
            # the forward LSE is within 2e-6 * max(1, |LSE|) (|LSE| about 12 here), which the
            # softmax term carries, plus the backward's own error; bf16 rounds the result
            bar = (2.0 ** -8 + 1e-4 if dtype == torch.bfloat16 else 5e-5) * scale
            assert np.all(np.abs(got - want) <= bar), (dtype, cols)
            assert np.all(big.grad.to(torch.float32).cpu().numpy()[:, cols:] == 0)
