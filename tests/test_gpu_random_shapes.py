"""A seeded sweep of random shapes through the C ABI, against the oracle.

Each case draws a dtype, a row count, a row length (spread over magnitudes,
1 to 400000, sometimes 0), a row padding, a misaligned start, a forced or
automatic schedule and sometimes a block / unroll / parts tuning within the
documented sets, plus rows of special values and dominated rows (one
maximum over many terms near half an fp32 ulp of the total); lse_forward and
lse_token_logprob (targets in and out of range) are compared with the
float64 oracle. A second sweep does the same for lse_forward_dim over random
[outer, n, inner] with forced or planned splits. The seeds are fixed, so every
run checks the same cases; each case is printed before it runs. A third
sweep runs lse_backward and lse_token_logprob_backward on random shapes with
padded and misaligned x and gradient rows (rows misaligned alike in x and
grad_x take the peeled 16-byte path, the others the element path), and
lse_backward_dim on random [outer, n, inner].

LSE_SWEEP_SEED=k (default 0) shifts every seed by 1000 k, for a wider sweep
run by hand; a list or range ("1-12", "3,5") runs each shift in the same
process. The default cases are the ones the suite always runs.
"""
import os

import numpy as np
import pytest

import oracle as oracle_mod
import workloads
from gpu_util import (DTYPE_CODE, SCHEDULES, compare, compare_dim_grad, compare_grad,
                      compare_logp, compare_token_grad, gpu_backward, gpu_dim_grad, gpu_lse,
                      gpu_token_backward, gpu_token_logprob, note)
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu

MAX_ELEMS = 3_000_000  # keeps each case's oracle call short


def _shifts(spec: str) -> list:
    out = []
    for part in spec.split(","):
        a, _, b = part.partition("-")
        out.extend(range(int(a), int(b or a) + 1))
    return out


SEEDS = [1000 * k for k in _shifts(os.environ.get("LSE_SWEEP_SEED", "0"))]


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


def log_int(rng, lo, hi):
    """An integer spread evenly over orders of magnitude in [lo, hi]."""
    v = np.exp(rng.uniform(np.log(lo), np.log(hi + 1)))
    return int(min(hi, max(lo, v)))


def dominated(rng, n):
    """n values with one maximum and the rest d = 14 to 22.5 below it, each
    term e^-d near or under half an fp32 ulp of the total: sums that drop
    small terms, and lazy references far below the maximum, show here."""
    base, d = rng.normal(0.0, 1.0), rng.uniform(14.0, 22.5)
    v = base - d + 0.01 * rng.normal(size=n)
    v[rng.integers(n)] = base
    return v


def make_rows(rng, rows, width, dtype, scale):
    v = rng.normal(0.0, scale, size=(rows, width)).astype(np.float32)
    if rows >= 1 and width > 0 and rng.random() < 0.5:
        for r in rng.integers(rows, size=min(rows, 3)):
            v[r] = dominated(rng, width)                   # one maximum over many tiny terms
    if rows >= 4 and width > 0 and rng.random() < 0.5:
        r = rng.integers(rows, size=4)
        v[r[0]] = -np.inf                                  # a row of -inf
        v[r[1], rng.integers(width)] = np.nan              # a NaN
        v[r[2], rng.integers(width)] = np.inf              # a +inf
        v[r[3]] += rng.choice([-1e3, 1e3, 3e9])            # large offsets, one beyond 2^30
    return workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v


def row_cases(seed, n):
    rng = np.random.default_rng(seed)
    for i in range(n):
        dtype = ["f32", "bf16"][rng.integers(2)]
        cols = 0 if rng.random() < 0.04 else log_int(rng, 1, 400_000)
        rows = log_int(rng, 1, 4000)
        while rows > 1 and rows * max(cols, 1) > MAX_ELEMS:
            rows //= 2
        pad = int(rng.choice([0, 0, 1, 5, 8, 24]))
        front = int(rng.choice([0, 0, 1, 2, 3]))
        sched = SCHEDULES[rng.integers(len(SCHEDULES))]
        tuning = (0, 0, 0, 0, 0)
        if rng.random() < 0.3:
            tuning = (int(rng.choice([0, 64, 128, 256, 512, 1024])), int(rng.choice([0, 4, 8])),
                      int(rng.choice([0, 2, 3, 7, 64])), int(rng.choice([0, 1, 8, 64])),
                      int(rng.choice([0, 1, 2, 4, 64])))
        scale = float(rng.choice([0.5, 3.0, 30.0]))
        yield i, dtype, rows, cols, pad, front, sched, tuning, scale, rng


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("block", range(8))
def test_random_rows(torch_gpu, handle, oracle, seed, block):
    for i, dtype, rows, cols, pad, front, sched, tuning, scale, rng in row_cases(seed + 100 + block, 50):
        full = make_rows(rng, rows, cols + pad, dtype, scale)
        x = full[:, :cols]
        what = (f"block {block} case {i}: {dtype} rows={rows} cols={cols} pad={pad} front={front} "
                f"schedule={sched} tuning={tuning}")
        note(what)
        got = gpu_lse(torch_gpu, handle, x, dtype, sched, pad_front=front, tuning=tuning)
        xc = np.ascontiguousarray(x)
        ref = oracle.lse(xc, dtype, threads=8)
        compare(got, ref, dtype, what)
        if cols > 0 and rows > 0:
            targets = rng.integers(-2, cols + 2, size=rows)
            logp, lse = gpu_token_logprob(torch_gpu, handle, x, targets, dtype, sched,
                                          pad_front=front, tuning=tuning)
            compare(lse, ref, dtype, what + " (token path LSE)")
            compare_logp(logp, oracle.token_logprob(xc, targets, dtype, threads=8), ref, dtype,
                         what + " (logp)")


def gpu_dim(torch, handle, x3, dtype, front, parts):
    outer, n, inner = x3.shape
    flat = np.zeros(front + x3.size, dtype=x3.dtype)
    flat[front:] = x3.ravel()
    t = torch.from_numpy(flat.view(np.int16 if dtype == "bf16" else np.int32)).to("cuda")
    out = torch.full((max(outer * inner, 1),), 123.0, dtype=torch.float32, device="cuda")
    B.lse_set_tuning(handle, 0, 0, parts, 0, 0)
    try:
        B.lse_forward_dim(handle, t.data_ptr() + front * x3.itemsize, DTYPE_CODE[dtype], outer,
                          n, inner, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        B.lse_set_tuning(handle, 0, 0, 0, 0, 0)
    return out.cpu().numpy()[: outer * inner]


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("block", range(6))
def test_random_dims(torch_gpu, handle, seed, block):
    rng = np.random.default_rng(seed + 200 + block)
    for i in range(30):
        dtype = ["f32", "bf16"][rng.integers(2)]
        outer, n, inner = log_int(rng, 1, 64), log_int(rng, 1, 60_000), log_int(rng, 1, 5000)
        while outer * n * inner > MAX_ELEMS:
            if n > 1:
                n //= 2
            else:
                inner = max(1, inner // 2)
        front = int(rng.choice([0, 0, 1]))
        parts = int(rng.choice([0, 0, 1, 2, 5, 64]))
        x = make_rows(rng, outer * n, inner, dtype, float(rng.choice([0.5, 3.0, 30.0])))
        x3 = x.reshape(outer, n, inner)
        if rng.random() < 0.5:                              # the same along the reduced axis
            o, i = rng.integers(outer), rng.integers(inner)
            col = dominated(rng, n).astype(np.float32)
            x3[o, :, i] = workloads.f32_to_bf16_bits(col) if dtype == "bf16" else col
        what = f"dim block {block} case {i}: {dtype} {x3.shape} front={front} parts={parts}"
        note(what)
        got = gpu_dim(torch_gpu, handle, x3, dtype, front, parts)
        compare(got, oracle_mod.lse_dim(x3, dtype, threads=8).ravel(), dtype, what)


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("block", range(3))
def test_random_dim_backward(torch_gpu, handle, seed, block):
    """lse_backward_dim on random [outer, n, inner] (the 16-byte and element
    paths, short rows cut into one-batch parts, forced splits), with x and
    grad_x sometimes misaligned, against the oracle; nothing outside grad_x
    is written."""
    rng = np.random.default_rng(seed + 500 + block)
    for i in range(20):
        dtype = ["f32", "bf16", "f16"][rng.integers(3)]
        outer, n, inner = log_int(rng, 1, 32), log_int(rng, 1, 60_000), log_int(rng, 1, 5000)
        while outer * n * inner > MAX_ELEMS // 2:
            if n > 1:
                n //= 2
            else:
                inner = max(1, inner // 2)
        front, gfront = int(rng.choice([0, 0, 1])), int(rng.choice([0, 0, 1]))
        parts = int(rng.choice([0, 0, 0, 1, 2, 7, 64]))
        v = rng.normal(0, float(rng.choice([0.5, 3.0, 30.0])), size=(outer, n, inner))
        v = v.astype(np.float32)
        x3 = (workloads.f32_to_bf16_bits(v) if dtype == "bf16" else
              workloads.f32_to_f16_bits(v) if dtype == "f16" else v)
        lse2 = oracle_mod.lse_dim(x3, dtype, threads=8).astype(np.float32)
        g2 = rng.normal(0, 2, size=(outer, inner)).astype(np.float32)
        what = (f"dim backward block {block} case {i}: {dtype} {x3.shape} front={front} "
                f"grad_front={gfront} parts={parts}")
        note(what)
        got, untouched = gpu_dim_grad(torch_gpu, handle, x3, lse2, g2, dtype, front, gfront, parts)
        assert untouched, what + ": bytes outside grad_x were written"
        compare_dim_grad(got, x3, lse2, g2, dtype, what)


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("block", range(4))
def test_random_backward(torch_gpu, handle, oracle, seed, block):
    rng = np.random.default_rng(seed + 300 + block)
    for i in range(30):
        dtype = ["f32", "bf16"][rng.integers(2)]
        cols = log_int(rng, 1, 300_000)
        rows = log_int(rng, 1, 3000)
        while rows > 1 and rows * cols > MAX_ELEMS // 2:
            rows //= 2
        pad = int(rng.choice([0, 0, 1, 8]))
        front, gpad, gfront = (int(rng.choice([0, 0, 1])), int(rng.choice([0, 0, 3, 8])),
                               int(rng.choice([0, 0, 2])))
        full = make_rows(rng, rows, cols + pad, dtype, float(rng.choice([0.5, 3.0, 30.0])))
        x = full[:, :cols]
        xc = np.ascontiguousarray(x)
        lse32 = oracle.lse(xc, dtype, threads=8).astype(np.float32)
        g = rng.normal(0, 2, size=rows).astype(np.float32)
        what = (f"backward block {block} case {i}: {dtype} rows={rows} cols={cols} pad={pad} "
                f"front={front} grad_pad={gpad} grad_front={gfront}")
        note(what)
        got, untouched = gpu_backward(torch_gpu, handle, x, lse32, g, dtype, pad_front=front,
                                      grad_pad=gpad, grad_front=gfront)
        assert untouched, what + ": bytes outside grad_x's rows were written"
        ref = oracle.softmax_grad(xc, lse32, g, dtype, threads=8)
        vals = (workloads.bf16_bits_to_f32(xc) if dtype == "bf16" else xc).astype(np.float64)
        with np.errstate(invalid="ignore"):
            d = vals - lse32.astype(np.float64)[:, None]
        compare_grad(got, ref, d, g, dtype, what)


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("block", range(3))
def test_random_token_backward(torch_gpu, handle, oracle, seed, block):
    """The token log-probability's backward on random shapes and layouts, with
    targets drawn in range and just outside it (rows of NaN)."""
    rng = np.random.default_rng(seed + 400 + block)
    for i in range(25):
        dtype = ["f32", "bf16"][rng.integers(2)]
        cols = log_int(rng, 1, 300_000)
        rows = log_int(rng, 1, 3000)
        while rows > 1 and rows * cols > MAX_ELEMS // 2:
            rows //= 2
        pad = int(rng.choice([0, 0, 1, 8]))
        front, gpad, gfront = (int(rng.choice([0, 0, 1])), int(rng.choice([0, 0, 3, 8])),
                               int(rng.choice([0, 0, 2])))
        full = make_rows(rng, rows, cols + pad, dtype, float(rng.choice([0.5, 3.0, 30.0])))
        x = full[:, :cols]
        xc = np.ascontiguousarray(x)
        lse32 = oracle.lse(xc, dtype, threads=8).astype(np.float32)
        g = rng.normal(0, 2, size=rows).astype(np.float32)
        targets = rng.integers(-1, cols + 1, size=rows)
        what = (f"token backward block {block} case {i}: {dtype} rows={rows} cols={cols} "
                f"pad={pad} front={front} grad_pad={gpad} grad_front={gfront}")
        note(what)
        got, untouched = gpu_token_backward(torch_gpu, handle, x, targets, lse32, g, dtype,
                                            pad_front=front, grad_pad=gpad, grad_front=gfront)
        assert untouched, what + ": bytes outside grad_x's rows were written"
        ref = oracle.token_logprob_grad(xc, targets, lse32, g, dtype, threads=8)
        soft = oracle.softmax_grad(xc, lse32, g, dtype, threads=8)
        vals = (workloads.bf16_bits_to_f32(xc) if dtype == "bf16" else xc).astype(np.float64)
        with np.errstate(invalid="ignore"):
            d = vals - lse32.astype(np.float64)[:, None]
        compare_token_grad(got, ref, soft, d, g, targets, dtype, what)
