"""GPU parity: the HIP library against the float64 oracle, through the C ABI.

* Every workload at a size the oracle finishes in seconds (a prefix of its
  rows that spans many tiles and a ragged tail), all rows, under every
  schedule.
* Every workload at full size, in the launch configuration the benchmark
  times (AUTO): every row against the oracle, and on all rows the bounds
  max <= LSE <= max + ln(#finite), exact -inf for empty rows, and config 5's
  closed form ln(sum of kept Dirichlet p).
"""
import math
import os

import numpy as np
import pytest

import workloads
from gpu_util import SCHEDULES, compare, gpu_lse, note
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu

PREFIX = {1: 64, 2: 40, 3: 12, 4: 3000, 5: 300_000}


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


@pytest.fixture(scope="module")
def prefixes():
    return {c: workloads.make(c, rows=n) for c, n in PREFIX.items()}


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_prefix_all_rows(torch_gpu, handle, oracle, prefixes, cfg, schedule):
    w = prefixes[cfg]
    if schedule == "split_row" and cfg == 5:
        w = workloads.make(5, rows=20_000)  # many launches of LSE_SPLIT_MAX_ROWS rows
    note(f"prefix cfg={cfg} rows={w.rows} schedule={schedule}")
    got = gpu_lse(torch_gpu, handle, w.x, w.dtype, schedule)
    ref = oracle.lse(w.x, w.dtype, threads=8)
    compare(got, ref, w.dtype, f"cfg{cfg} prefix {schedule}")


@pytest.fixture(scope="module")
def full_outputs(torch_gpu, handle):
    """Each workload at full size through AUTO; keeps the host input for checks."""
    cache = {}

    def get(cfg):
        if cfg not in cache:
            cache.clear()
            w = workloads.make(cfg, aux=(cfg == 5))
            note(f"full cfg={cfg} shape={w.x.shape} dtype={w.dtype}")
            got = gpu_lse(torch_gpu, handle, w.x, w.dtype, "auto")
            cache[cfg] = (w, got)
        return cache[cfg]
    return get


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_every_row(torch_gpu, oracle, full_outputs, cfg):
    """Every row of the full workload against the oracle (run on all host
    cores), in the launch configuration the benchmark times."""
    w, got = full_outputs(cfg)
    ref = oracle.lse(w.x, w.dtype, threads=len(os.sched_getaffinity(0)))
    compare(got, ref, w.dtype, f"cfg{cfg} full, every row")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_bounds_every_row(torch_gpu, full_outputs, cfg):
    """max <= LSE <= max + ln(#finite) on every row, within the tolerance."""
    torch = torch_gpu
    w, got = full_outputs(cfg)
    x = torch.from_numpy(w.x.view(np.int16) if w.dtype == "bf16" else w.x).to("cuda")
    if w.dtype == "bf16":
        x = x.view(torch.bfloat16)
    mx = x.amax(dim=1).double().cpu().numpy()
    cnt = torch.isfinite(x).sum(dim=1).double().cpu().numpy()
    del x
    tol = {"f32": 2e-6, "bf16": 1e-5}[w.dtype]
    dead = cnt == 0
    assert np.all(got[dead] == -np.inf)
    g = got[~dead].astype(np.float64)
    slack = tol * np.maximum(1.0, np.abs(mx[~dead]))
    assert np.all(g >= mx[~dead] - slack)
    assert np.all(g <= mx[~dead] + np.log(cnt[~dead]) + slack)


def test_full_size_config5_closed_form(torch_gpu, full_outputs):
    """Rows of fp32(ln p) with p ~ Dirichlet: LSE = ln(sum of kept p) within tol + rounding."""
    w, got = full_outputs(5)
    keep = w.aux["keep"].copy()
    keep[w.aux["allneg"]] = False
    p = w.aux["p"]
    dead = ~keep.any(axis=1)
    assert np.array_equal(np.isneginf(got), dead)
    mass = np.where(keep, p, 0.0).sum(axis=1)
    delta = np.where(keep, np.abs(w.x.astype(np.float64) - np.log(p)), 0.0).max(axis=1)
    live = ~dead
    err = np.abs(got[live].astype(np.float64) - np.log(mass[live]))
    assert np.all(err <= delta[live] + 2e-6 * np.maximum(1.0, np.abs(np.log(mass[live]))))


def test_logsumexp_tensor_api(torch_gpu):
    """The torch-facing helper on a padded bf16 view and an fp32 tensor."""
    import oracle as orc
    import row_wise_log_amd as lib
    torch = torch_gpu
    g = torch.Generator(device="cpu").manual_seed(3)
    base = (torch.randn(300, 5000, generator=g) * 3).to(torch.bfloat16)
    view = base[:, :4093]
    note("logsumexp tensor api")
    dev = base.to("cuda")[:, :4093]  # row stride 5000: a padded view
    assert dev.stride(0) == 5000
    got = lib.logsumexp(dev).cpu().numpy()
    bits = view.contiguous().view(torch.int16).numpy().view(np.uint16)
    compare(got, orc.lse(bits, "bf16"), "bf16", "tensor api bf16 view")
    f = torch.randn(33, 70000, generator=g) * 10
    got = lib.logsumexp(f.to("cuda")).cpu().numpy()
    compare(got, orc.lse(f.numpy(), "f32"), "f32", "tensor api f32")
    assert math.isclose(float(got[0]), float(torch.logsumexp(f[0].double(), 0)), rel_tol=2e-6)
