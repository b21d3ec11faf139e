"""The entry points under HIP graph capture and on concurrent streams.

lse_forward, lse_token_logprob, lse_backward, lse_forward_dim and
lse_backward_dim allocate nothing and synchronise nothing, and the split
schedules' arrival counters are reset by the kernels themselves, so a caller
may capture the calls into a graph and replay it. One graph holds every
schedule (register rows, a workgroup per row, split rows, the token
log-probability, the backward pass, a split LSE over a non-last axis and two
backward passes over it); it is replayed several times with new
inputs written by eager work in between, and every replay is compared bit for
bit with the same calls made eagerly. A second test runs split-row and split
non-last-axis calls on two handles on two streams at once (one handle per
stream, as the header asks) and compares every result with a serial run; a
third does the same through the torch-level functions, which keep one handle
per (device, stream).
"""
import numpy as np
import pytest

import oracle as oracle_mod
from gpu_util import compare, note
from row_wise_log_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _bits(torch, t):
    return t.detach().cpu().numpy().view(np.uint32).copy()


class Calls:
    """Inputs, handles and one output set per `run` target."""

    def __init__(self, torch, seed):
        self.torch = torch
        rng = np.random.default_rng(seed)
        dev = "cuda"
        self.rng = rng
        self.shapes = {"a": (64, 128256, torch.bfloat16), "b": (8, 300_000, torch.float32),
                       "c": (10_000, 100, torch.float32), "d": (37, 5000, torch.float32),
                       "e": (50_000, 256, torch.float32)}
        self.x = {k: torch.empty(r, c, dtype=dt, device=dev) for k, (r, c, dt) in self.shapes.items()}
        self.targets = torch.from_numpy(rng.integers(0, 128256, size=64)).to(dev)
        self.lse_d = torch.empty(37, device=dev)
        self.g_d = torch.from_numpy(rng.normal(0, 1, size=37).astype(np.float32)).to(dev)
        # lse and grad_out of x["e"] and x["c"] over their first axis (the dim backward)
        self.lse_e, self.lse_c = torch.empty(256, device=dev), torch.empty(100, device=dev)
        self.g_e = torch.from_numpy(rng.normal(0, 1, size=256).astype(np.float32)).to(dev)
        self.g_c = torch.from_numpy(rng.normal(0, 1, size=100).astype(np.float32)).to(dev)
        self.h = B.lse_create(0)
        self.h_split = B.lse_create(0)
        B.lse_set_schedule(self.h_split, "split_row")
        self.refill()

    def refill(self):
        torch = self.torch
        for k, (r, c, dt) in self.shapes.items():
            v = self.rng.normal(0, 3, size=(r, c)).astype(np.float32)
            self.x[k].copy_(torch.from_numpy(v).to(dt))
        s = torch.cuda.current_stream().cuda_stream
        B.lse_forward(self.h, self.x["d"].data_ptr(), B.LSE_DTYPE_F32, 37, 5000, 5000,
                      self.lse_d.data_ptr(), s)
        B.lse_forward_dim(self.h, self.x["e"].data_ptr(), B.LSE_DTYPE_F32, 1, 50_000, 256,
                          self.lse_e.data_ptr(), s)
        B.lse_forward_dim(self.h, self.x["c"].data_ptr(), B.LSE_DTYPE_F32, 1, 10_000, 100,
                          self.lse_c.data_ptr(), s)

    def outputs(self):
        torch = self.torch
        return {"a": torch.empty(64, device="cuda"), "b": torch.empty(8, device="cuda"),
                "c": torch.empty(10_000, device="cuda"), "lp": torch.empty(64, device="cuda"),
                "lse_a": torch.empty(64, device="cuda"),
                "grad": torch.empty(37, 5000, device="cuda"), "dim": torch.empty(256, device="cuda"),
                "dgrad_e": torch.empty(50_000, 256, device="cuda"),
                "dgrad_c": torch.empty(10_000, 100, device="cuda")}

    def run(self, o):
        s = self.torch.cuda.current_stream().cuda_stream
        x = self.x
        B.lse_forward(self.h, x["a"].data_ptr(), B.LSE_DTYPE_BF16, 64, 128256, 128256,
                      o["a"].data_ptr(), s)
        B.lse_forward(self.h_split, x["b"].data_ptr(), B.LSE_DTYPE_F32, 8, 300_000, 300_000,
                      o["b"].data_ptr(), s)
        B.lse_forward(self.h, x["c"].data_ptr(), B.LSE_DTYPE_F32, 10_000, 100, 100,
                      o["c"].data_ptr(), s)
        B.lse_token_logprob(self.h, x["a"].data_ptr(), B.LSE_DTYPE_BF16, 64, 128256, 128256,
                            self.targets.data_ptr(), o["lp"].data_ptr(), o["lse_a"].data_ptr(), s)
        B.lse_backward(self.h, x["d"].data_ptr(), B.LSE_DTYPE_F32, 37, 5000, 5000,
                       self.lse_d.data_ptr(), self.g_d.data_ptr(), o["grad"].data_ptr(), 5000, s)
        # 50000 x 256 over the first axis: 2 tiles of 32 column groups, j split
        B.lse_forward_dim(self.h, x["e"].data_ptr(), B.LSE_DTYPE_F32, 1, 50_000, 256,
                          o["dim"].data_ptr(), s)
        # the backward over the first axis: split tiles, and short rows in one-batch parts
        B.lse_backward_dim(self.h, x["e"].data_ptr(), B.LSE_DTYPE_F32, 1, 50_000, 256,
                           self.lse_e.data_ptr(), self.g_e.data_ptr(), o["dgrad_e"].data_ptr(), s)
        B.lse_backward_dim(self.h, x["c"].data_ptr(), B.LSE_DTYPE_F32, 1, 10_000, 100,
                           self.lse_c.data_ptr(), self.g_c.data_ptr(), o["dgrad_c"].data_ptr(), s)

    def close(self):
        self.torch.cuda.synchronize()
        B.lse_destroy(self.h)
        B.lse_destroy(self.h_split)


def test_graph_replays_match_eager(torch_gpu):
    torch = torch_gpu
    c = Calls(torch, seed=21)
    try:
        og, oe = c.outputs(), c.outputs()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm up off the default stream, as capture wants
            c.run(og)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        note("graph capture of every entry point")
        with torch.cuda.graph(graph):
            c.run(og)
        torch.cuda.synchronize()
        for rep in range(4):
            c.refill()                    # eager work between replays
            torch.cuda.synchronize()
            note(f"graph replay {rep}")
            graph.replay()
            torch.cuda.synchronize()
            c.run(oe)                     # the same calls, eagerly
            torch.cuda.synchronize()
            for k in og:
                assert np.array_equal(_bits(torch, og[k]), _bits(torch, oe[k])), (rep, k)
            # and one result against the oracle, so the replays compute the LSE
            ref = oracle_mod.lse(c.x["b"].cpu().numpy(), "f32", threads=8)
            compare(og["b"].cpu().numpy(), ref, "f32", f"graph replay {rep} split rows")
        del graph
    finally:
        c.close()


def test_two_handles_on_two_streams(torch_gpu):
    torch = torch_gpu
    rng = np.random.default_rng(22)
    n = 8
    xs = [torch.from_numpy(rng.normal(0, 3, size=(16, 262_144)).astype(np.float32)).cuda()
          for _ in range(n)]
    ds = [torch.from_numpy(rng.normal(0, 3, size=(40_000, 512)).astype(np.float32)).cuda()
          for _ in range(n)]
    ha, hb = B.lse_create(0), B.lse_create(0)
    try:
        B.lse_set_schedule(ha, "split_row")
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        out_a = [torch.empty(16, device="cuda") for _ in range(n)]
        out_b = [torch.empty(512, device="cuda") for _ in range(n)]
        note("two handles, two streams")
        for rep in range(3):
            for i in range(n):
                B.lse_forward(ha, xs[i].data_ptr(), B.LSE_DTYPE_F32, 16, 262_144, 262_144,
                              out_a[i].data_ptr(), sa.cuda_stream)
                B.lse_forward_dim(hb, ds[i].data_ptr(), B.LSE_DTYPE_F32, 1, 40_000, 512,
                                  out_b[i].data_ptr(), sb.cuda_stream)
            torch.cuda.synchronize()
            for i in range(n):
                ra = oracle_mod.lse(xs[i].cpu().numpy(), "f32", threads=8)
                compare(out_a[i].cpu().numpy(), ra, "f32", f"stream a rep {rep} call {i}")
                rb = oracle_mod.lse_dim(ds[i].cpu().numpy().reshape(1, 40_000, 512), "f32",
                                        threads=8).ravel()
                compare(out_b[i].cpu().numpy(), rb, "f32", f"stream b rep {rep} call {i}")
    finally:
        torch.cuda.synchronize()
        B.lse_destroy(ha)
        B.lse_destroy(hb)


def test_package_calls_on_two_streams(torch_gpu):
    """The torch-level functions keep one library handle per (device,
    stream), so calls issued on two streams at once never share a split
    workspace: split-row and split non-last-axis shapes, alternated between
    two streams with no synchronisation between them, give exactly the
    results of the same calls made one at a time."""
    import row_wise_log_amd as R
    torch = torch_gpu
    rng = np.random.default_rng(21)
    xs = [torch.from_numpy(rng.normal(0, 3, size=(8, 300_000)).astype(np.float32)).cuda()
          for _ in range(4)]                            # few long rows: the split-row schedule
    ds = [torch.from_numpy(rng.normal(0, 3, size=(20_000, 64)).astype(np.float32)).cuda()
          for _ in range(4)]                            # a tall [n, inner]: split over n
    torch.cuda.synchronize()
    want = [R.logsumexp(x) for x in xs] + [R.logsumexp_dim(d, 0) for d in ds]
    torch.cuda.synchronize()
    want = [_bits(torch, w) for w in want]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        note(f"package calls on two streams, repeat {rep}")
        got = []
        for i in range(4):
            with torch.cuda.stream(s1 if i % 2 == 0 else s2):
                got.append(R.logsumexp(xs[i]))
        for i in range(4):
            with torch.cuda.stream(s2 if i % 2 == 0 else s1):
                got.append(R.logsumexp_dim(ds[i], 0))
        torch.cuda.synchronize()
        for k, (g, w) in enumerate(zip(got, want)):
            assert np.array_equal(_bits(torch, g), w), (rep, k)


def test_package_helpers_captured_on_a_fresh_stream(torch_gpu):
    """The torch-level helpers inside torch.cuda.graph on a new stream: with
    no handle prepared for it, the helper raises a clear error before any HIP
    call (a handle cannot be made while capturing); after prepare(stream) the
    captured logsumexp / token_logprob / logsumexp_autograd forward replay
    correctly, four times, with new inputs written eagerly in between."""
    torch = torch_gpu
    import row_wise_log_amd as lib
    rng = np.random.default_rng(5)
    x = torch.empty(24, 90_000, device="cuda")                       # split rows (fp32)
    xb = torch.empty(600, 128256, dtype=torch.bfloat16, device="cuda")  # a workgroup per row
    t = torch.from_numpy(rng.integers(0, 128256, size=600)).to("cuda")
    lib.logsumexp(torch.zeros(2, 8, device="cuda"))  # code objects loaded eagerly elsewhere
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    note("package helpers: capture without prepare must raise")
    g0 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g0, stream=s):
        with pytest.raises(RuntimeError, match="prepare"):
            lib.logsumexp(x)
        _ = x.sum(dim=1)  # the capture ends with ordinary work in it
    del g0
    lib.prepare(s)
    g = torch.cuda.CUDAGraph()
    note("package helpers: capture after prepare")
    with torch.cuda.graph(g, stream=s):
        out_a = lib.logsumexp(x)
        lp, lse_b = lib.token_logprob(xb, t, return_lse=True)
    torch.cuda.synchronize()
    for rep in range(4):
        va = rng.normal(0, 3, size=(24, 90_000)).astype(np.float32)
        vb = rng.normal(0, 2, size=(600, 128256)).astype(np.float32)
        x.copy_(torch.from_numpy(va))
        xb.copy_(torch.from_numpy(vb).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = xb.view(torch.int16).cpu().numpy().view(np.uint16)
        compare(out_a.cpu().numpy(), oracle_mod.lse(va, "f32", threads=8), "f32",
                f"captured logsumexp replay {rep}")
        ref_b = oracle_mod.lse(bits, "bf16", threads=8)
        compare(lse_b.cpu().numpy(), ref_b, "bf16", f"captured token_logprob lse replay {rep}")
        ref_lp = oracle_mod.token_logprob(bits, t.cpu().numpy(), "bf16", threads=8)
        got_lp = lp.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got_lp - ref_lp) <= 1e-5 * np.maximum(1.0, np.abs(ref_b))), rep
    del g
    lib.release(s)


def test_package_handle_cache_is_bounded(torch_gpu):
    """Eager helper calls on more streams than the cache keeps: at most
    MAX_HANDLES_PER_DEVICE unpinned handles stay per device, and every call
    still computes the right result."""
    torch = torch_gpu
    import row_wise_log_amd as lib
    x = torch.full((3, 1000), 2.0, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(lib.MAX_HANDLES_PER_DEVICE + 4)]
    for st in streams:
        with torch.cuda.stream(st):
            out = lib.logsumexp(x)
        st.synchronize()
        assert np.allclose(out.cpu().numpy(), 2.0 + np.log(1000.0), rtol=2e-6)
        loose = [k for k in lib._handles if k[0] == 0 and k not in lib._pinned]
        assert len(loose) <= lib.MAX_HANDLES_PER_DEVICE
    for st in streams:
        lib.release(st)


def test_package_helpers_from_several_host_threads(torch_gpu):
    """Helper calls from four host threads, each on its own stream, all at
    once: every stream gets exactly one handle, no two streams share one, and
    every result matches the oracle."""
    import threading

    torch = torch_gpu
    import row_wise_log_amd as lib
    rng = np.random.default_rng(77)
    vals = [rng.normal(0, 3, size=(40, 70_000)).astype(np.float32) for _ in range(4)]
    xs = [torch.from_numpy(v).to("cuda") for v in vals]
    streams = [torch.cuda.Stream() for _ in vals]
    outs, errors = [None] * len(vals), []
    start = threading.Barrier(len(vals))

    def work(i):
        try:
            start.wait()
            with torch.cuda.stream(streams[i]):
                for _ in range(20):
                    outs[i] = lib.logsumexp(xs[i])
            streams[i].synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(vals))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    keys = [(0, st.cuda_stream) for st in streams]
    assert all(k in lib._handles for k in keys)
    assert len({lib._handles[k] for k in keys}) == len(keys)
    for i, v in enumerate(vals):
        compare(outs[i].cpu().numpy(), oracle_mod.lse(v, "f32", threads=8), "f32",
                f"host thread {i}")
    for st in streams:
        lib.release(st)
