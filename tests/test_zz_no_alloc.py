"""GPU: lse_forward_noalloc (no handle, no allocation, per-device scratch)
against lse_forward on the same inputs, through the C ABI.

Each case makes two calls in a row, the second on a smaller input, and
checks both outputs against lse_forward's (bit for bit: the same plan and
kernels) and against the float64 oracle at the LSE bar (2e-6 fp32, 1e-5 bf16,
times max(1, |LSE|)). The split-row shapes use the scratch's pairs and
counters; the second, smaller call reuses what the first left there.
"""
import numpy as np
import pytest

import workloads
from gpu_util import DTYPE_CODE, compare, note, upload
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _run(torch, fn, x: np.ndarray, dtype: str) -> np.ndarray:
    rows, cols = x.shape
    t, ptr, stride = upload(torch, x)
    out = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    fn(ptr, DTYPE_CODE[dtype], rows, cols, stride, out.data_ptr(),
       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del t
    return out.cpu().numpy()


# (workload, rows of the first call, rows of the second, schedule the planner picks)
CASES = [
    (2, 40, 8, B.LSE_SCHED_SPLIT_ROW),      # bf16 vocabulary rows: 32 then 64 parts per row
    (1, 64, 16, B.LSE_SCHED_SPLIT_ROW),     # fp32 [64, 32000]: 16 parts per row, then more
    (5, 300_000, 1000, B.LSE_SCHED_ROWS_PER_WAVE),
    (4, 3000, 100, B.LSE_SCHED_ROW_PER_WG),
]


@pytest.mark.parametrize("cfg,first,second,sched", CASES)
def test_noalloc_matches_lse_forward(torch_gpu, oracle, cfg, first, second, sched):
    torch = torch_gpu
    w = workloads.make(cfg, rows=first)
    h = B.lse_create(0)
    try:
        for rows in (first, second):
            x = np.ascontiguousarray(w.x[:rows])
            p = B.lse_plan(DTYPE_CODE[w.dtype], rows, w.cols, w.cols, 0, 256, 0)
            assert p["schedule"] == sched, p
            note(f"noalloc cfg={cfg} rows={rows} (then lse_forward)")
            got = _run(torch, B.lse_forward_noalloc, x, w.dtype)
            ref_gpu = _run(torch, lambda *a: B.lse_forward(h, *a), x, w.dtype)
            assert np.array_equal(got.view(np.uint32), ref_gpu.view(np.uint32)), \
                f"cfg{cfg} rows={rows}: lse_forward_noalloc differs from lse_forward"
            ref = oracle.lse(x, w.dtype, threads=8)
            compare(got, ref, w.dtype, f"noalloc cfg{cfg} rows={rows}")
    finally:
        torch.cuda.synchronize()
        B.lse_destroy(h)


def test_noalloc_alternating_split_inputs(torch_gpu, oracle):
    """Split-row calls that alternate two inputs differing by +5 in every
    element, back to back on one stream: a merge that read a stale pair of
    the previous call from the scratch would be off by about 5."""
    torch = torch_gpu
    rng = np.random.default_rng(11)
    a = rng.normal(0, 3, size=(24, 90_000)).astype(np.float32)
    b = a + np.float32(5.0)
    refs = [oracle.lse(a, "f32", threads=8), oracle.lse(b, "f32", threads=8)]
    devs = [torch.from_numpy(a).to("cuda"), torch.from_numpy(b).to("cuda")]
    assert B.lse_plan(B.LSE_DTYPE_F32, 24, 90_000, 90_000, 0, 256, 0)["schedule"] == \
        B.LSE_SCHED_SPLIT_ROW
    calls = 100
    outs = torch.empty((calls, 24), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    note("noalloc alternating split inputs")
    for i in range(calls):
        B.lse_forward_noalloc(devs[i % 2].data_ptr(), B.LSE_DTYPE_F32, 24, 90_000, 90_000,
                              outs[i].data_ptr(), stream)
    torch.cuda.synchronize()
    got = outs.cpu().numpy()
    for i in range(calls):
        compare(got[i], refs[i % 2], "f32", f"noalloc alternating call {i}")


def test_noalloc_alternating_part_counts(torch_gpu, oracle):
    """Split-row calls through the shared scratch whose plans cut rows into
    16, 64 and 32 parts, back to back: each call's (row, part) slots overlap
    the previous call's at other offsets, so each must leave what it used
    clear. Every output equals the first of its shape bit for bit and
    matches the oracle."""
    torch = torch_gpu
    shapes = [(64, 32000), (8, 128256), (40, 70_000)]
    devs, refs, parts = [], [], []
    for k, (rows, cols) in enumerate(shapes):
        x = np.random.default_rng(60 + k).normal(0, 3, size=(rows, cols)).astype(np.float32)
        refs.append(oracle.lse(x, "f32", threads=8))
        devs.append(torch.from_numpy(x).to("cuda"))
        plan = B.lse_plan(B.LSE_DTYPE_F32, rows, cols, cols, devs[-1].data_ptr(), 256, 0)
        assert plan["schedule"] == B.LSE_SCHED_SPLIT_ROW
        parts.append(plan["parts"])
    assert len(set(parts)) == len(shapes), parts
    calls = 90
    outs = [torch.empty((calls // len(shapes), rows), device="cuda") for rows, _ in shapes]
    stream = torch.cuda.current_stream().cuda_stream
    note(f"noalloc alternating part counts {parts}")
    for i in range(calls):
        k = i % len(shapes)
        rows, cols = shapes[k]
        B.lse_forward_noalloc(devs[k].data_ptr(), B.LSE_DTYPE_F32, rows, cols, cols,
                              outs[k][i // len(shapes)].data_ptr(), stream)
    torch.cuda.synchronize()
    for k, (rows, cols) in enumerate(shapes):
        o = outs[k].cpu().numpy()
        assert np.all(o.view(np.uint32) == o[0].view(np.uint32)), (rows, cols)
        compare(o[0], refs[k], "f32", f"noalloc alternating parts {rows}x{cols}")
