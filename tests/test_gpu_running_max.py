"""GPU parity on rows whose running maximum moves while the row streams.

The streaming schedules keep, per lane, a reference that may trail the true
running maximum by up to 32*ln2 and is only refreshed when a batch's sum
against it passes 2^32 (or when no finite maximum is known yet, or the
reference lies beyond +-2^30). These rows make that refresh happen early,
late, often, right at the threshold, or never, and are compared with the
float64 oracle under every streaming schedule.
"""
import numpy as np
import pytest

import workloads
from gpu_util import compare, gpu_lse, note
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu

LN2 = float(np.log(2.0))


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


def moving_max_rows(cols: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    j = np.arange(cols, dtype=np.float64)
    rows = []
    rows.append(0.01 * j)                                 # steady climb, max grows by 0.01*cols
    rows.append(-0.01 * j)                                # first elements hold the maximum
    rows.append(40.0 * np.sin(j / 997.0))                 # climbs and falls repeatedly
    for jump in (20.0, 22.0, 22.18, 22.2, 23.0, 50.0, 88.0, 1e4):
        r = rng.normal(0, 1, cols)                        # one late jump above the rest
        r[cols - 3] = jump
        rows.append(r)
        r = rng.normal(0, 1, cols)                        # the same jump mid-row
        r[cols // 2] = jump
        rows.append(r)
    r = rng.normal(0, 1, cols)
    r[: cols // 2] = -np.inf                              # no finite maximum in the first half
    rows.append(r)
    r = np.full(cols, -np.inf)
    r[-1] = 3.0                                           # one finite element, the last
    rows.append(r)
    r = rng.normal(0, 1, cols)
    r[-1] = 2.0e9                                         # late maximum beyond 2^30
    rows.append(r)
    r = rng.normal(0, 1, cols) - 2.0e9                    # every element beyond -2^30
    rows.append(r)
    r = np.full(cols, -2.0e9)
    r[-2] = -2.0e9 + 256.0                                # late rise, still beyond -2^30
    rows.append(r)
    r = np.full(cols, -1.2e9)
    r[cols // 3] = -1.0e9                                 # the reference crosses back inside
    r[-1] = 5.0
    rows.append(r)
    r = rng.normal(0, 1, cols)
    r[-5] = np.inf                                        # late +inf
    rows.append(r)
    r = rng.normal(0, 1, cols)
    r[-7] = np.nan                                        # late NaN
    rows.append(r)
    r = rng.normal(0, 1, cols)
    r[-7] = np.nan                                        # late NaN after a late +inf
    r[-9] = np.inf
    rows.append(r)
    r = rng.normal(0, 3, cols) + np.where(j < cols // 2, 0.0, 30.0)   # a step of +30
    rows.append(r)
    r = rng.normal(0, 3, cols) + 25.0 * np.floor(j / 4096.0)          # a staircase of +25 steps
    rows.append(r)
    return np.asarray(rows, dtype=np.float32)


@pytest.mark.parametrize("cols", [4097, 32001, 128257, 300_003])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_moving_maximum(torch_gpu, handle, oracle, dtype, cols):
    v = moving_max_rows(cols, seed=cols)
    x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
    ref = oracle.lse(x, dtype)
    for sched in ["auto", "row_per_wg", "split_row"]:
        note(f"moving max dtype={dtype} cols={cols} schedule={sched}")
        got = gpu_lse(torch_gpu, handle, x, dtype, sched)
        compare(got, ref, dtype, f"moving max {dtype} cols={cols} {sched}")


def test_threshold_jumps_exactly(torch_gpu, handle, oracle):
    """A constant row with one element k*ln2 above it, for k around 32 (the
    refresh threshold of 2^32 in base 2), at every position of a batch."""
    cols = 70_000
    rows = []
    for k in (31.0, 31.9, 32.0, 32.1, 33.0, 38.0, 64.0):
        for pos in (0, 1, 7, 8, 4095, 4096, cols // 2, cols - 8, cols - 1):
            r = np.zeros(cols, dtype=np.float32)
            r[pos] = np.float32(k * LN2)
            rows.append(r)
    v = np.asarray(rows)
    for dtype, x in [("f32", v), ("bf16", workloads.f32_to_bf16_bits(v))]:
        ref = oracle.lse(x, dtype)
        for sched in ["row_per_wg", "split_row"]:
            note(f"threshold jumps dtype={dtype} schedule={sched}")
            compare(gpu_lse(torch_gpu, handle, x, dtype, sched), ref, dtype,
                    f"threshold jumps {dtype} {sched}")


def trailing_reference_rows(cols: int, seed: int) -> np.ndarray:
    """Rows whose LSE lies near zero while a lane's reference trails the
    maximum by up to 32*ln2 (22.18): the first elements a lane folds sit d
    below a later maximum near 0.3, for d up to just under the refresh
    threshold, so the lane's sum grows to about 2^(d*log2 e)."""
    rng = np.random.default_rng(seed)
    rows = []
    for d in (8.0, 12.0, 16.68, 20.0, 21.5, 22.1):
        r = np.full(cols, -np.float32(d) + 0.3, dtype=np.float64)
        r[cols // 2 + 1] = 0.3                             # one maximum, mid-row
        rows.append(r)
        r = -d + 0.3 + 0.01 * rng.normal(size=cols)
        r[-2] = 0.3                                        # near the end
        rows.append(r)
        r = np.full(cols, -np.inf)
        r[0] = -d + 0.3                                    # the first element far below
        r[1:5] = [0.47797355, -20.94657898, -26.51913834, -48.59749603][: min(4, cols - 1)]
        rows.append(r)
    return np.asarray(rows, dtype=np.float32)


@pytest.mark.parametrize("cols", [5, 40, 4097, 70_001])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reference_far_below_the_maximum(torch_gpu, handle, oracle, dtype, cols):
    """The finish takes log2 of a sum of up to 2^38 without losing absolute
    accuracy (it splits off the sum's binary exponent first), and no result
    falls below the row's maximum by more than that bound. The remaining error on these rows
    (results near 0.3-0.5) is the fp32 rounding of the largest term's
    exponent x*log2 e - c, which is below 32 while the reference trails:
    half an ulp, 2^-20, is 6.6e-7 in the result; with the exponential's and
    the logarithm's own rounding the bound is 1e-6, half the fp32 bar. (Taking
    log2 of the whole sum left 2.1e-6 on such a row.) Rows start 0-3 elements
    past a 16-byte boundary, so the first elements are also folded singly (a
    misaligned head) before the vectors."""
    v = trailing_reference_rows(cols, seed=cols)
    x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
    ref = oracle.lse(x, dtype)
    xv = workloads.bf16_bits_to_f32(x) if dtype == "bf16" else x
    mx = xv.astype(np.float64).max(axis=1)
    for sched, tuning in [("row_per_wg", (0, 0, 0, 0, 0)), ("row_per_wg", (128, 0, 0, 0, 0)),
                          ("split_row", (0, 0, 0, 0, 0)), ("auto", (0, 0, 0, 0, 0))]:
        for front in (0, 1, 3):
            what = f"trailing reference {dtype} cols={cols} {sched} {tuning} front={front}"
            note(what)
            got = gpu_lse(torch_gpu, handle, x, dtype, sched, pad_front=front, tuning=tuning)
            err = np.abs(got.astype(np.float64) - ref)
            assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(ref))), (what, float(err.max()))
            assert np.all(got.astype(np.float64) >= mx - 1e-6 * np.maximum(1.0, np.abs(mx))), what
