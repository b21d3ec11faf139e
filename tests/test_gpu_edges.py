"""GPU edge cases: ragged and tiny widths, padded and misaligned rows, special
values, huge magnitudes, the largest row, determinism and repeated calls.

Every case runs under every schedule (AUTO and the three forced ones) and is
compared with the float64 oracle, or with a closed form where the oracle
would take too long.
"""
import math

import numpy as np
import pytest

import golden_cases
import workloads
from gpu_util import SCHEDULES, compare, gpu_lse, note
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu

COLS = [0, 1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 33, 255, 257, 1023, 1025, 4095, 4097, 8193,
        32001, 128257]
LAYOUTS = ["contiguous", "padded", "misaligned"]


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


def make_rows(dtype, rows, cols, layout, seed):
    """Random rows with special rows mixed in; returns (array view, pad_front)."""
    rng = np.random.default_rng(seed)
    pad = {"contiguous": 0, "padded": 5, "misaligned": 0}[layout]
    v = rng.normal(0, 5, size=(rows, cols + pad)).astype(np.float32)
    if cols:
        v[3 % rows] = -np.inf                       # empty sum
        v[5 % rows, rng.integers(cols)] = np.nan    # NaN anywhere
        v[7 % rows, rng.integers(cols)] = np.inf    # +inf
        v[11 % rows] = 2.5                          # constant
        v[13 % rows, : cols // 2] = -np.inf         # half -inf
        v[17 % rows] -= 200.0                       # far below zero
    x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
    x = x[:, :cols] if pad else x
    front = 1 if layout == "misaligned" else 0
    return x, front


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_sweep(torch_gpu, handle, oracle, dtype, cols, layout):
    x, front = make_rows(dtype, 37, cols, layout, seed=cols * 7 + len(layout))
    ref = oracle.lse(x, dtype)
    for sched in SCHEDULES:
        note(f"edge dtype={dtype} cols={cols} layout={layout} schedule={sched}")
        got = gpu_lse(torch_gpu, handle, x, dtype, sched, pad_front=front)
        compare(got, ref, dtype, f"{dtype} cols={cols} {layout} {sched}")


@pytest.mark.parametrize("rows", [1, 2, 63, 64, 65, 1023, 1025, 3000])
def test_row_counts(torch_gpu, handle, oracle, rows):
    """Row counts around the wavefront, group and split-batch boundaries."""
    for dtype, cols in [("f32", 16), ("bf16", 24), ("f32", 3000), ("bf16", 20000)]:
        x, _ = make_rows(dtype, rows, cols, "contiguous", seed=rows + cols)
        ref = oracle.lse(x, dtype, threads=8)
        for sched in SCHEDULES:
            note(f"rows={rows} dtype={dtype} cols={cols} schedule={sched}")
            compare(gpu_lse(torch_gpu, handle, x, dtype, sched), ref, dtype,
                    f"rows={rows} {dtype} cols={cols} {sched}")


@pytest.mark.parametrize("tuning", [(64, 4, 0), (64, 8, 5), (128, 4, 0), (128, 8, 2),
                                    (256, 4, 0), (256, 8, 3), (512, 4, 0), (512, 8, 0),
                                    (1024, 4, 0), (1024, 8, 64), (256, 4, 1)])
def test_streaming_tunings(torch_gpu, handle, oracle, tuning):
    """Every block/unroll instance of the streaming kernels, split and not."""
    for dtype in ["f32", "bf16"]:
        x, front = make_rows(dtype, 9, 100_003, "misaligned", seed=sum(tuning))
        ref = oracle.lse(x, dtype)
        for sched in ["row_per_wg", "split_row"]:
            note(f"tuning={tuning} dtype={dtype} schedule={sched}")
            got = gpu_lse(torch_gpu, handle, x, dtype, sched, pad_front=front, tuning=tuning)
            compare(got, ref, dtype, f"tuning {tuning} {dtype} {sched}")


def test_golden_cases(torch_gpu, handle):
    for case in golden_cases.load():
        x = case["x"]
        for sched in SCHEDULES:
            note(f"golden {case['name']} schedule={sched}")
            got = gpu_lse(torch_gpu, handle, x, case["dtype"], sched)
            compare(got, case["out"], case["dtype"], f"golden {case['name']} {sched}")


@pytest.mark.parametrize("cols", [5, 300, 70_001])
def test_huge_magnitudes(torch_gpu, handle, oracle, cols):
    """Row maxima beyond 2^126 take the natural-units pass; the result is max + ln(count)."""
    rng = np.random.default_rng(cols)
    v = rng.normal(0, 1, size=(6, cols)).astype(np.float32)
    v[0] = 3.0e38
    v[1] = -3.0e38
    v[2, ::2] = 2.0e38
    v[3] = -1.0e38
    v[3, -1] = 1.0e38
    v[4, : cols // 2] = -3.3e38
    v[4, cols // 2:] = -3.2e38
    v[5] = rng.uniform(-3e38, 3e38, size=cols).astype(np.float32)
    for dtype, x in [("f32", v), ("bf16", workloads.f32_to_bf16_bits(v))]:
        ref = oracle.lse(x, dtype)
        for sched in SCHEDULES:
            note(f"huge cols={cols} dtype={dtype} schedule={sched}")
            compare(gpu_lse(torch_gpu, handle, x, dtype, sched), ref, dtype,
                    f"huge {dtype} cols={cols} {sched}")


def test_empty_inputs(torch_gpu, handle):
    torch = torch_gpu
    out = torch.full((4,), 7.0, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    B.lse_forward(handle, 0, B.LSE_DTYPE_F32, 0, 10, 10, out.data_ptr(), stream)
    B.lse_forward(handle, 0, B.LSE_DTYPE_F32, 0, 10, 10, 0, stream)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    B.lse_forward(handle, 0, B.LSE_DTYPE_BF16, 4, 0, 0, out.data_ptr(), stream)
    torch.cuda.synchronize()
    assert torch.all(out == -math.inf)


def test_deterministic_and_schedules_agree(torch_gpu, handle):
    """Bitwise-equal repeats per schedule; schedules agree within the tolerance."""
    w = workloads.make(1)
    outs = {}
    for sched in SCHEDULES:
        note(f"determinism schedule={sched}")
        a = gpu_lse(torch_gpu, handle, w.x, "f32", sched)
        b = gpu_lse(torch_gpu, handle, w.x, "f32", sched)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), sched
        outs[sched] = a
    for sched in SCHEDULES[1:]:
        compare(outs[sched], outs["auto"].astype(np.float64), "f32", f"{sched} vs auto")


def test_split_counters_reset_over_many_calls(torch_gpu, handle, oracle):
    """The split-row arrival counters reset themselves: 300 calls give one answer."""
    torch = torch_gpu
    x = np.random.default_rng(1).normal(0, 3, size=(48, 50_000)).astype(np.float32)
    ref = oracle.lse(x, "f32")
    dev = torch.from_numpy(x).to("cuda")
    outs = torch.empty((300, 48), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    B.lse_set_schedule(handle, "split_row")
    try:
        note("split counters: 300 calls")
        for i in range(300):
            B.lse_forward(handle, dev.data_ptr(), B.LSE_DTYPE_F32, 48, 50_000, 50_000,
                          outs[i].data_ptr(), stream)
        torch.cuda.synchronize()
    finally:
        B.lse_set_schedule(handle, "auto")
    o = outs.cpu().numpy()
    assert np.all(o.view(np.uint32) == o[0].view(np.uint32))
    compare(o[0], ref, "f32", "split repeated")


def test_side_stream(torch_gpu, handle, oracle):
    torch = torch_gpu
    x = np.random.default_rng(2).normal(0, 3, size=(700, 3000)).astype(np.float32)
    dev = torch.from_numpy(x).to("cuda")
    s = torch.cuda.Stream()
    out = torch.empty(700, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        note("side stream")
        B.lse_forward(handle, dev.data_ptr(), B.LSE_DTYPE_F32, 700, 3000, 3000, out.data_ptr(),
                      s.cuda_stream)
    s.synchronize()
    compare(out.cpu().numpy(), oracle.lse(x, "f32"), "f32", "side stream")


def test_largest_row(torch_gpu, handle):
    """One bf16 row of 2^31 - 1 elements (4 GiB): three constant thirds with a
    closed form ln(a + b e^-2 + c e^1); byte offsets pass 2^31 and 2^32."""
    torch = torch_gpu
    n = (1 << 31) - 1
    x = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    a = n // 3
    b = n // 3
    c = n - a - b
    x[:a] = 0.0
    x[a:a + b] = -2.0
    x[a + b:] = 1.0
    def closed_form(i0, length):
        """ln sum exp over x[i0 : i0 + length] of the three constant thirds."""
        n0 = max(0, min(a, i0 + length) - i0)
        n1 = max(0, min(a + b, i0 + length) - max(a, i0))
        n2 = length - n0 - n1
        return math.log(n0 + n1 * math.exp(-2.0) + n2 * math.exp(1.0))

    half = (n - 1) // 2
    want = [closed_form(0, n), closed_form(1, half), closed_form(1 + half, half)]
    out = torch.empty(3, device="cuda")
    for sched in SCHEDULES:
        note(f"largest row schedule={sched}")
        B.lse_set_schedule(handle, sched)
        try:
            stream = torch.cuda.current_stream().cuda_stream
            B.lse_forward(handle, x.data_ptr(), B.LSE_DTYPE_BF16, 1, n, n, out.data_ptr(), stream)
            # the same buffer as two rows of (n - 1) / 2 elements starting one element in;
            # the second row ends at the buffer's last element
            B.lse_forward(handle, x.data_ptr() + 2, B.LSE_DTYPE_BF16, 2, half, half,
                          out.data_ptr() + 4, stream)
            torch.cuda.synchronize()
        finally:
            B.lse_set_schedule(handle, "auto")
        got = out.cpu().numpy().astype(np.float64)
        for g, w in zip(got, want):
            assert abs(g - w) <= 1e-5 * abs(w), (sched, got, want)
    del x


# (dtype, rows, cols, layout, expected automatic plan: block, parts)
FEW_LONG_ROWS = [
    ("bf16", 1, 128256, "contiguous", 64, 64),     # one batch per lane: 64 parts of 64 threads
    ("bf16", 3, 128257, "misaligned", 64, 64),     # head peel in part 0, tail in the last part
    ("f32", 8, 1 << 20, "contiguous", 128, 64),    # 128 wavefronts per row: wider workgroups
    ("f32", 1, 1 << 22, "padded", 512, 64),        # the widest split workgroup
    ("bf16", 95, 65539, "padded", 64, 16),         # 128 KiB rows just under 3/8 of the CUs
    ("bf16", 40, 262144, "misaligned", 64, 32),    # 512 KiB rows, a share of 26 wavefronts, 32
    ("f32", 64, 32000, "contiguous", 64, 16),      # the small fp32 vocabulary workload
    ("bf16", 257, 524288, "padded", 256, 4),       # just over one 1 MiB row per CU: quarters
    ("f32", 320, 262144, "misaligned", 256, 4),    # 5/4 rows per CU, the band's upper end
]


@pytest.mark.parametrize("dtype,rows,cols,layout,block,parts", FEW_LONG_ROWS)
def test_few_long_rows_automatic_split(torch_gpu, handle, oracle, dtype, rows, cols, layout, block,
                                       parts):
    """The automatic plans for few long rows: the split the planner picks for
    the shape (checked against the expected block and part count) matches the
    oracle, with special rows mixed in and misaligned or padded rows."""
    x, front = make_rows(dtype, rows, cols, layout, seed=rows * 31 + cols)
    code = B.LSE_DTYPE_BF16 if dtype == "bf16" else B.LSE_DTYPE_F32
    esize = 2 if dtype == "bf16" else 4
    stride = x.strides[0] // x.itemsize if rows > 1 else cols
    p = B.lse_plan(code, rows, cols, stride, front * esize, 256, 0)
    assert (p["schedule"], p["block"], p["parts"]) == (B.LSE_SCHED_SPLIT_ROW, block, parts), p
    ref = oracle.lse(x, dtype, threads=8)
    note(f"few long rows {dtype} {rows}x{cols} {layout}: split {block}x{parts}")
    got = gpu_lse(torch_gpu, handle, x, dtype, "auto", pad_front=front)
    compare(got, ref, dtype, f"few long rows {dtype} {rows}x{cols} {layout}")


@pytest.mark.parametrize("dtype,rows,cols", [("f32", 64, 32000), ("bf16", 7, 300_001)])
def test_split_alternating_inputs(torch_gpu, handle, oracle, dtype, rows, cols):
    """Back-to-back split-row calls alternate two inputs that differ by +5 in
    every element: a part merged with a stale pair from the previous call would
    be off by ~5. Every call must match its own input's oracle value."""
    torch = torch_gpu
    rng = np.random.default_rng(rows)
    a = rng.normal(0, 3, size=(rows, cols)).astype(np.float32)
    b = a + np.float32(5.0)
    if dtype == "bf16":
        a, b = workloads.f32_to_bf16_bits(a), workloads.f32_to_bf16_bits(b)
    refs = [oracle.lse(a, dtype, threads=8), oracle.lse(b, dtype, threads=8)]
    view = (lambda v: torch.from_numpy(v.view(np.int16)).to("cuda")) if dtype == "bf16" else \
        (lambda v: torch.from_numpy(v).to("cuda"))
    devs = [view(a), view(b)]
    calls = 200
    outs = torch.empty((calls, rows), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    code = B.LSE_DTYPE_BF16 if dtype == "bf16" else B.LSE_DTYPE_F32
    for sched in ["split_row", "auto"]:
        B.lse_set_schedule(handle, sched)
        try:
            note(f"split alternating {dtype} {rows}x{cols} schedule={sched}")
            for i in range(calls):
                B.lse_forward(handle, devs[i % 2].data_ptr(), code, rows, cols, cols,
                              outs[i].data_ptr(), stream)
            torch.cuda.synchronize()
        finally:
            B.lse_set_schedule(handle, "auto")
        o = outs.cpu().numpy()
        for i in range(calls):
            assert np.array_equal(o[i].view(np.uint32), o[i % 2].view(np.uint32)), (sched, i)
        compare(o[0], refs[0], dtype, f"alternating a {sched}")
        compare(o[1], refs[1], dtype, f"alternating b {sched}")


def test_split_alternating_part_counts(torch_gpu, handle, oracle):
    """Back-to-back split-row calls on one handle whose plans cut rows into
    different numbers of parts, so that each call's (row, part) slots overlap
    the previous call's at other offsets: every call must leave the slots it
    used clear for the next, whatever its layout. Each output must equal the
    first of its shape bit for bit and match the oracle."""
    torch = torch_gpu
    shapes = [("f32", 64, 32000), ("bf16", 8, 128256), ("f32", 3, 300_001), ("bf16", 40, 70_000)]
    devs, refs, codes, plans = [], [], [], []
    for k, (dtype, rows, cols) in enumerate(shapes):
        v = np.random.default_rng(40 + k).normal(0, 3, size=(rows, cols)).astype(np.float32)
        x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
        refs.append(oracle.lse(x, dtype, threads=8))
        devs.append(torch.from_numpy(x.view(np.int16) if dtype == "bf16" else x).to("cuda"))
        codes.append(B.LSE_DTYPE_BF16 if dtype == "bf16" else B.LSE_DTYPE_F32)
        plans.append(B.lse_plan(codes[-1], rows, cols, cols, devs[-1].data_ptr(), 256, 0))
    assert all(p["schedule"] == 3 for p in plans), plans
    assert len({p["parts"] for p in plans}) > 1, plans
    calls = 120
    outs = [torch.empty((calls // len(shapes), rows), device="cuda") for _, rows, _ in shapes]
    stream = torch.cuda.current_stream().cuda_stream
    note(f"split alternating part counts {[p['parts'] for p in plans]}")
    for i in range(calls):
        k = i % len(shapes)
        _, rows, cols = shapes[k]
        B.lse_forward(handle, devs[k].data_ptr(), codes[k], rows, cols, cols,
                      outs[k][i // len(shapes)].data_ptr(), stream)
    torch.cuda.synchronize()
    for k, (dtype, rows, cols) in enumerate(shapes):
        o = outs[k].cpu().numpy()
        assert np.all(o.view(np.uint32) == o[0].view(np.uint32)), (dtype, rows, cols)
        compare(o[0], refs[k], dtype, f"alternating parts {dtype} {rows}x{cols}")
