"""GPU parity of the LSE over a non-last axis, lse_forward_dim, against the
float64 oracle (the reduced axis moved last, then the row oracle).

Shapes [outer, n, inner] with vector and single-column paths, the split of
n across workgroups (forced and planned, in batches of tiles), special and
huge-magnitude columns (also in narrow tiles, whose lanes share columns in
the end-of-workgroup merge), n == 0, inner == 1 (the row path), a misaligned
base, two workloads and [1, 1000000, inner] arrays of one or two column groups
reduced over their first axis at full size, and the package's
torch-tensor entry against torch.logsumexp in float64.
"""
import numpy as np
import pytest

import oracle as oracle_mod
import workloads
from gpu_util import DTYPE_CODE, compare, note
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


def gpu_dim(torch, handle, x3: np.ndarray, dtype: str, front: int = 0, parts: int = 0):
    outer, n, inner = x3.shape
    flat = np.zeros(front + x3.size, dtype=x3.dtype)
    flat[front:] = x3.ravel()
    t = torch.from_numpy(flat.view(np.int16 if dtype == "bf16" else np.int32)).to("cuda")
    out = torch.full((max(outer * inner, 1),), 123.0, dtype=torch.float32, device="cuda")
    B.lse_set_tuning(handle, 0, 0, parts, 0, 0)
    try:
        B.lse_forward_dim(handle, t.data_ptr() + front * x3.itemsize, DTYPE_CODE[dtype], outer, n,
                          inner, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        B.lse_set_tuning(handle, 0, 0, 0, 0, 0)
    return out.cpu().numpy()[: outer * inner].reshape(outer, inner)


def make(shape, dtype, seed, scale=4.0):
    v = np.random.default_rng(seed).normal(0, scale, size=shape).astype(np.float32)
    return workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v


SHAPES = [(1, 8192, 4096), (64, 1000, 32), (3, 5, 7), (2, 100_000, 3), (128, 17, 1024),
          (1, 1, 100), (10, 300, 1), (7, 33, 12), (1, 3, 65), (16, 257, 40), (1, 64, 4 * 64 * 300)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shapes(torch_gpu, handle, dtype, shape):
    x = make(shape, dtype, seed=sum(shape))
    ref = oracle_mod.lse_dim(x, dtype, threads=8)
    for front in (0, 1):
        note(f"dim shape={shape} dtype={dtype} front={front}")
        got = gpu_dim(torch_gpu, handle, x, dtype, front=front)
        compare(got.ravel(), ref.ravel(), dtype, f"dim {shape} {dtype} front={front}")


@pytest.mark.parametrize("parts", [1, 2, 7, 64])
def test_forced_parts(torch_gpu, handle, parts):
    for dtype in ["f32", "bf16"]:
        x = make((3, 5000, 256), dtype, seed=parts)
        ref = oracle_mod.lse_dim(x, dtype, threads=8)
        note(f"dim forced parts={parts} dtype={dtype}")
        compare(gpu_dim(torch_gpu, handle, x, dtype, parts=parts).ravel(), ref.ravel(), dtype,
                f"parts={parts} {dtype}")


def test_split_in_tile_batches(torch_gpu, handle):
    """More tiles than one split launch holds: several launches, counters reused."""
    x = make((1, 40, 4 * 64 * 1100), "f32", seed=5)   # 1100 tiles of 64 column vectors
    ref = oracle_mod.lse_dim(x, "f32", threads=8)
    for parts in (2, 5):
        note(f"dim tile batches parts={parts}")
        compare(gpu_dim(torch_gpu, handle, x, "f32", parts=parts).ravel(), ref.ravel(), "f32",
                f"tile batches parts={parts}")


def test_special_and_huge_columns(torch_gpu, handle):
    rng = np.random.default_rng(8)
    for dtype in ["f32", "bf16"]:
        v = rng.normal(0, 2, size=(2, 3000, 64)).astype(np.float32)
        v[0, :, 0] = -np.inf                     # a column of only -inf
        v[0, 1234, 1] = np.nan                   # NaN
        v[0, 2999, 2] = np.inf                   # +inf, last step
        v[1, :, 3] = 7.0                         # constant: 7 + ln 3000
        v[1, :1500, 4] = -np.inf                 # half -inf
        v[1, 2000, 5] = 2.0e9                    # maximum beyond 2^30: natural units
        v[1, :, 6] -= 2.0e9                      # every element beyond -2^30
        v[0, :, 7] = 3.0e38                      # near the largest float
        v[0, 0, 8] = 60.0                        # first step holds the maximum
        v[0, 2999, 9] = 60.0                     # last step holds the maximum
        x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
        ref = oracle_mod.lse_dim(x, dtype, threads=8)
        for parts in (0, 1, 3):
            note(f"dim special columns dtype={dtype} parts={parts}")
            compare(gpu_dim(torch_gpu, handle, x, dtype, parts=parts).ravel(), ref.ravel(), dtype,
                    f"special {dtype} parts={parts}")


@pytest.mark.parametrize("dtype,inner", [("f32", 4), ("f32", 8), ("bf16", 8), ("bf16", 16),
                                         ("f32", 3), ("bf16", 5)])
def test_special_values_in_narrow_tiles(torch_gpu, handle, dtype, inner):
    """Rows of one or two 16-byte groups (or a few single columns): each
    workgroup reads 32 to 256 steps of j at once, and several lanes share a
    column in the end-of-workgroup merge. Special columns as above, split and
    unsplit, with and without a misaligned base."""
    rng = np.random.default_rng(inner)
    v = rng.normal(0, 2, size=(2, 5000, inner)).astype(np.float32)
    v[0, :, 0] = -np.inf
    v[0, 4321, 1] = np.nan
    v[1, 4999, 0] = np.inf
    v[1, :2500, 1] = -np.inf
    v[1, 17, 2] = 2.0e9
    v[0, 0, 2] = 60.0
    v[0, 4999, inner - 1] = 60.0
    x = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
    ref = oracle_mod.lse_dim(x, dtype, threads=8)
    for parts in (0, 1, 3):
        for front in (0, 1):
            note(f"dim narrow special dtype={dtype} inner={inner} parts={parts} front={front}")
            compare(gpu_dim(torch_gpu, handle, x, dtype, parts=parts, front=front).ravel(),
                    ref.ravel(), dtype, f"narrow special {dtype} inner={inner} parts={parts}")


@pytest.mark.parametrize("dtype,inner", [("bf16", 8), ("f32", 4), ("bf16", 7)])
def test_long_narrow_full_size(torch_gpu, handle, dtype, inner):
    """[1, 1000000, inner]: one column group per j-row, so one tile whose 256
    lanes read 256 steps of j per load, split into about one workgroup per
    CU; every output against the oracle."""
    x = make((1, 1_000_000, inner), dtype, seed=inner)
    ref = oracle_mod.lse_dim(x, dtype, threads=8)
    note(f"dim long narrow dtype={dtype} inner={inner}")
    compare(gpu_dim(torch_gpu, handle, x, dtype).ravel(), ref.ravel(), dtype,
            f"long narrow {dtype} inner={inner}")


def test_empty_reduction(torch_gpu, handle):
    x = np.zeros((3, 0, 9), np.float32)
    note("dim n=0")
    got = gpu_dim(torch_gpu, handle, x, "f32")
    assert np.all(got == -np.inf)
    B.lse_forward_dim(handle, 0, B.LSE_DTYPE_F32, 0, 5, 5, 0,
                      torch_gpu.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("cfg", [2, 4])
def test_workload_first_axis_full_size(torch_gpu, handle, cfg):
    """A workload reduced over its first axis (outer = 1, n = rows, inner = cols)."""
    w = workloads.make(cfg)
    x3 = w.x.reshape(1, w.rows, w.cols)
    ref = oracle_mod.lse_dim(x3, w.dtype, threads=16)
    note(f"dim workload {cfg} over axis 0")
    compare(gpu_dim(torch_gpu, handle, x3, w.dtype).ravel(), ref.ravel(), w.dtype,
            f"workload {cfg} axis 0")


def test_package_logsumexp_dim(torch_gpu):
    import row_wise_log_amd as R
    torch = torch_gpu
    rng = np.random.default_rng(12)
    v = rng.normal(0, 3, size=(6, 50, 7, 33)).astype(np.float32)
    xt = torch.from_numpy(v).cuda()
    for d in range(4):
        note(f"package logsumexp_dim dim={d}")
        got = R.logsumexp_dim(xt, d).cpu().numpy().astype(np.float64)
        want = torch.logsumexp(torch.from_numpy(v).double(), dim=d).numpy()
        assert got.shape == want.shape
        assert np.all(np.abs(got - want) <= 2e-6 * np.maximum(1.0, np.abs(want))), d


def test_package_keepdim_and_adjacent_axes(torch_gpu):
    """logsumexp_dim against torch.logsumexp in float64 on the CPU: keepdim,
    negative axes, tuples of adjacent axes (one reduced axis of a contiguous
    tensor), every axis of a rank-1 tensor, and the refusal of other tuples."""
    import row_wise_log_amd as R
    torch = torch_gpu
    rng = np.random.default_rng(13)
    v = rng.normal(0, 3, size=(4, 6, 5, 7)).astype(np.float32)
    xt = torch.from_numpy(v).cuda()
    xc = torch.from_numpy(v).double()
    for dim in [0, -1, 2, (1, 2), (0, 1), (2, 3), (0, 1, 2, 3), (-2, -1)]:
        for keepdim in (False, True):
            note(f"package logsumexp_dim dim={dim} keepdim={keepdim}")
            got = R.logsumexp_dim(xt, dim, keepdim=keepdim).cpu().double()
            want = torch.logsumexp(xc, dim=dim, keepdim=keepdim)
            assert got.shape == want.shape, (dim, keepdim, got.shape, want.shape)
            assert torch.all((got - want).abs() <= 2e-6 * torch.clamp(want.abs(), min=1.0)), (dim, keepdim)
    one = torch.from_numpy(v[0, 0, 0]).cuda()
    assert abs(float(R.logsumexp_dim(one, 0)) - float(torch.logsumexp(one.double().cpu(), 0))) < 2e-5
    with pytest.raises(NotImplementedError):
        R.logsumexp_dim(xt, (0, 2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trailing_reference_columns(torch_gpu, handle, dtype):
    """Columns whose elements lie up to 22 below one maximum near 0.3. Where
    a lane's reference trails the maximum (long columns) its sum reaches
    2^31, which the shared finish handles; where every lane holds one
    element (n = 64 over 3 columns), the merge adds one partial near 1 and
    63 of 5.7e-8, each under half an ulp of the total, which only a
    compensated sum keeps (a plain one lost 1.7e-6). The result stays within
    1e-6 of the oracle, split and unsplit, vector and single-column paths."""
    rng = np.random.default_rng(5)
    for n, inner in ((4096, 64), (300, 40), (64, 3)):
        cols = []
        for d in (8.0, 16.68, 21.5, 22.1):
            c = np.full(n, 0.3 - d) + 0.01 * rng.normal(size=n)
            c[n // 2 + 1] = 0.3
            cols.append(c)
        v = np.tile(np.asarray(cols).T, (1, -(-inner // len(cols))))[:, :inner]
        v = v.astype(np.float32).reshape(1, n, inner)
        x3 = workloads.f32_to_bf16_bits(v) if dtype == "bf16" else v
        ref = oracle_mod.lse_dim(x3, dtype)
        for parts in (0, 1, 3):
            for front in (0, 1):
                note(f"trailing reference columns {dtype} n={n} inner={inner} parts={parts} front={front}")
                got = gpu_dim(torch_gpu, handle, x3, dtype, front=front, parts=parts)
                err = np.abs(got.astype(np.float64) - ref)
                assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(ref))), (n, inner, parts, front,
                                                                            float(err.max()))
