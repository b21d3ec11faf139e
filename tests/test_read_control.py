"""The control kernels that bench.py times beside the LSE kernels.

It must read every byte it is given, or the rate it reports would flatter
the device and understate how close the LSE kernels come to it: each chunk's
XOR of 32-bit words is compared with numpy's over the same words, for ragged
sizes, more chunks than vectors, every block size, and the headline
workload's exact geometry (512 chunks of one 256512-byte row each, 512
threads). The copy control must move every byte to the same offset and
write nothing else. The argument checks of both run on the host before any
HIP call, so they are tested without a GPU.
"""
import numpy as np
import pytest

from row_wise_log_amd import read_control as RC


def bounds(nvec: int, chunks: int, g: int) -> tuple[int, int]:
    """Chunk g's vectors: q = nvec // chunks each, one more for the first
    nvec % chunks chunks."""
    q, r = divmod(nvec, chunks)
    v0 = g * q + min(g, r)
    return v0, v0 + q + (1 if g < r else 0)


def expected(words: np.ndarray, chunks: int) -> np.ndarray:
    nvec = words.size // 4
    out = np.zeros(chunks, dtype=np.uint32)
    for g in range(chunks):
        v0, v1 = bounds(nvec, chunks, g)
        if v1 > v0:
            out[g] = np.bitwise_xor.reduce(words[4 * v0: 4 * v1])
    return out


def test_expected_helper_by_brute_force():
    """The numpy reference itself, against a word-by-word loop."""
    rng = np.random.default_rng(0)
    w = rng.integers(0, 2 ** 32, size=4 * 37, dtype=np.uint32)
    for chunks in (1, 5, 37, 50):
        nvec = 37
        # the chunks tile the vectors in order, without gaps or overlaps
        spans = [bounds(nvec, chunks, g) for g in range(chunks)]
        assert spans[0][0] == 0 and spans[-1][1] == nvec
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
        want = []
        for g in range(chunks):
            acc = 0
            for v in range(*spans[g]):
                for k in range(4):
                    acc ^= int(w[4 * v + k])
            want.append(acc)
        assert list(expected(w, chunks)) == want


@pytest.mark.parametrize("args", [
    dict(nbytes=15, chunks=1, block=256),          # not whole vectors
    dict(nbytes=-16, chunks=1, block=256),
    dict(nbytes=16, chunks=0, block=256),
    dict(nbytes=16, chunks=1, block=100),          # not a supported block
    dict(nbytes=16, chunks=1, block=2048),
    dict(nbytes=16, chunks=2 ** 31, block=256),
    dict(nbytes=16, chunks=1, block=256, x=8),     # x not 16-byte aligned
    dict(nbytes=16, chunks=1, block=256, x=0),     # null
    dict(nbytes=16, chunks=1, block=256, out=0),
    dict(nbytes=16, chunks=1, block=256, out=6),   # out not 4-byte aligned
])
def test_argument_checks_on_host(args):
    a = dict(x=1 << 20, out=1 << 21)
    a.update(args)
    with pytest.raises(ValueError):
        RC.lse_control_read(a["x"], a["nbytes"], a["chunks"], a["block"], a["out"], 0)


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def run(torch, data: np.ndarray, chunks: int, block: int) -> np.ndarray:
    x = torch.from_numpy(data.view(np.int32)).cuda()
    out = torch.full((chunks,), -1, dtype=torch.int32, device="cuda")
    RC.lse_control_read(x.data_ptr(), data.nbytes, chunks, block, out.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


@pytest.mark.gpu
@pytest.mark.parametrize("block", [64, 128, 256, 512, 1024])
def test_every_word_is_read(torch_gpu, block):
    rng = np.random.default_rng(block)
    for nvec in (0, 1, 3, 4 * block - 1, 4 * block, 4 * block + 1, 8 * block + 5, 50_001):
        words = rng.integers(0, 2 ** 32, size=4 * nvec, dtype=np.uint32)
        for chunks in (1, 3, 64, nvec + 7):
            print(f"read control block={block} nvec={nvec} chunks={chunks}", flush=True)
            if nvec == 0:
                data = np.zeros(4, dtype=np.uint32)   # a valid pointer, zero bytes read
                x = torch_gpu.from_numpy(data.view(np.int32)).cuda()
                out = torch_gpu.full((chunks,), -1, dtype=torch_gpu.int32, device="cuda")
                RC.lse_control_read(x.data_ptr(), 0, chunks, block, out.data_ptr(),
                                    torch_gpu.cuda.current_stream().cuda_stream)
                torch_gpu.cuda.synchronize()
                assert np.all(out.cpu().numpy() == 0)
                continue
            got = run(torch_gpu, words, chunks, block)
            assert np.array_equal(got, expected(words, chunks)), (block, nvec, chunks)


@pytest.mark.gpu
def test_headline_geometry(torch_gpu):
    """The bf16 [512, 128256] workload as bench.py times it: 512 chunks, one
    row each, 512 threads."""
    import workloads
    w = workloads.make(2)
    words = np.ascontiguousarray(w.x).view(np.uint32).ravel()
    print("read control workload 2 geometry", flush=True)
    got = run(torch_gpu, words, 512, 512)
    rows = words.reshape(512, -1)
    assert np.array_equal(got, np.bitwise_xor.reduce(rows, axis=1))


@pytest.mark.parametrize("args", [
    dict(nbytes=15),                       # not whole vectors
    dict(nbytes=-16),
    dict(chunks=0),
    dict(block=96),
    dict(src=8),                           # not 16-byte aligned
    dict(dst=24),
    dict(src=0),
    dict(dst=0),
    dict(src=1 << 20, dst=(1 << 20) + 4096, nbytes=8192),   # overlapping ranges
    dict(src=(1 << 20) + 4096, dst=1 << 20, nbytes=8192),
])
def test_copy_argument_checks_on_host(args):
    a = dict(src=1 << 20, dst=1 << 24, nbytes=4096, chunks=4, block=256)
    a.update(args)
    with pytest.raises(ValueError):
        RC.lse_control_copy(a["src"], a["dst"], a["nbytes"], a["chunks"], a["block"], 0)


@pytest.mark.gpu
@pytest.mark.parametrize("block", [64, 256, 1024])
def test_copy_moves_every_byte(torch_gpu, block):
    torch = torch_gpu
    rng = np.random.default_rng(100 + block)
    for nvec in (1, 4 * block - 1, 4 * block, 8 * block + 5, 50_001):
        for chunks in (1, 3, -(-nvec // 1024), nvec + 7):
            print(f"copy control block={block} nvec={nvec} chunks={chunks}", flush=True)
            data = rng.integers(0, 2 ** 32, size=4 * nvec, dtype=np.uint32)
            src = torch.from_numpy(data.view(np.int32)).cuda()
            guard = 64   # words of canary on each side of the destination
            dst = torch.full((4 * nvec + 2 * guard,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
            RC.lse_control_copy(src.data_ptr(), dst[guard:].data_ptr(), 16 * nvec, chunks, block,
                                torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            out = dst.cpu().numpy().view(np.uint32)
            assert np.array_equal(out[guard:guard + 4 * nvec], data), (block, nvec, chunks)
            assert np.all(out[:guard] == 0x5A5A5A5A) and np.all(out[guard + 4 * nvec:] == 0x5A5A5A5A)


@pytest.mark.parametrize("args", [
    dict(nbytes=4095, grid=1),          # not whole 4 KiB iterations
    dict(nbytes=-4096, grid=1),
    dict(nbytes=4096, grid=0),
])
def test_rows_argument_checks_on_host(args):
    with pytest.raises(ValueError):
        RC.lse_control_rows(16, args["nbytes"], args["grid"], True, 16, 0)
    with pytest.raises(ValueError):
        RC.lse_control_rows(0, 4096, 1, True, 16, 0)          # NULL x
    with pytest.raises(ValueError):
        RC.lse_control_rows(8, 4096, 1, True, 16, 0)          # x not 16-byte aligned


@pytest.mark.gpu
@pytest.mark.parametrize("iters,grid", [(1, 1), (7, 2), (1000, 3), (4096, 512)])
def test_rows_control_reads_every_row(torch_gpu, iters, grid):
    """The row control's per-row XOR (store) and per-wavefront XOR (no store)
    against numpy: every 64-byte row read, every row's word stored."""
    torch = torch_gpu
    rng = np.random.default_rng(iters)
    words = rng.integers(0, 2 ** 32, size=iters * 1024, dtype=np.uint32)
    x = torch.from_numpy(words.view(np.int32)).cuda()
    rows = iters * 64
    per_row = np.bitwise_xor.reduce(words.reshape(rows, 16), axis=1)
    out = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    RC.lse_control_rows(x.data_ptr(), words.nbytes, grid, True, out.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), per_row)
    nwaves = grid * 4
    out = torch.full((nwaves,), -1, dtype=torch.int32, device="cuda")
    RC.lse_control_rows(x.data_ptr(), words.nbytes, grid, False, out.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = np.zeros(nwaves, dtype=np.uint32)
    for it in range(iters):  # iteration it (64 rows) belongs to wavefront it % nwaves
        want[it % nwaves] ^= np.bitwise_xor.reduce(per_row[it * 64:(it + 1) * 64])
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
