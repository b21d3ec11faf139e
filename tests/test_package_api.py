"""The Python package's argument checks, and its refusal to run without the
library, on the CPU (no device call is reached)."""
import pytest

torch = pytest.importorskip("torch")

import row_wise_log_amd as R  # noqa: E402
from row_wise_log_amd import binding as B  # noqa: E402


def test_logsumexp_rejects_bad_tensors():
    with pytest.raises(ValueError, match="2-D"):
        R.logsumexp(torch.zeros(4))
    with pytest.raises(ValueError, match="2-D"):
        R.logsumexp(torch.zeros(2, 3, 4))
    with pytest.raises(ValueError, match="GPU"):
        R.logsumexp(torch.zeros(4, 8))
    with pytest.raises(ValueError, match="GPU"):
        R.logsumexp_autograd(torch.zeros(4, 8))


def test_token_logprob_rejects_bad_tensors():
    with pytest.raises(ValueError, match="2-D"):
        R.token_logprob(torch.zeros(8), torch.zeros(8, dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU"):
        R.token_logprob(torch.zeros(4, 8), torch.zeros(4, dtype=torch.int64))


def test_logsumexp_dim_rejects_bad_tensors():
    with pytest.raises(TypeError, match="unsupported dtype"):
        R.logsumexp_dim(torch.zeros(2, 3, dtype=torch.float64), 0)
    with pytest.raises(TypeError, match="unsupported dtype"):
        R.logsumexp_dim(torch.zeros(2, 3, dtype=torch.int32), 1)
    with pytest.raises(ValueError, match="contiguous GPU"):
        R.logsumexp_dim(torch.zeros(2, 3), 1)
    with pytest.raises(ValueError, match="contiguous GPU"):
        R.logsumexp_dim(torch.zeros(2, 3), (0, 1), keepdim=True)


def test_missing_library_is_an_error(tmp_path):
    """No fallback: loading a library that is not there raises."""
    saved = B._lib
    B._lib = None
    try:
        with pytest.raises(RuntimeError, match="no fallback"):
            B.load(tmp_path / "liblse_amd.so")
    finally:
        B._lib = saved


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message."""
    import json
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parent.parent
    proc = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=300, cwd=root)
    assert proc.returncode == 2
    msg = json.loads(proc.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_logsumexp_dim_checks_its_axes():
    """Axes are checked as torch.logsumexp checks them, before anything
    touches a device: out of range, repeated, or not adjacent."""
    torch = pytest.importorskip("torch")
    import row_wise_log_amd as R
    x = torch.zeros(2, 3, 4)
    for bad, err in ((3, IndexError), (-4, IndexError), ((0, 5), IndexError),
                     ((1, 1), ValueError), ((0, -3), ValueError), ((), ValueError),
                     ((0, 2), NotImplementedError)):
        with pytest.raises(err):
            R.logsumexp_dim(x, bad)
    with pytest.raises(ValueError):        # valid axes, but a CPU tensor
        R.logsumexp_dim(x, (1, 2))


def test_gradient_paths_refuse_what_they_cannot_differentiate():
    """With an input that requires a gradient (grad mode on), the plain helpers
    take their autograd variants; out= and return_lse=True, which those cannot
    serve, raise instead of silently dropping the gradient (before any device
    call)."""
    x = torch.zeros(4, 8, requires_grad=True)
    with pytest.raises(RuntimeError, match="out="):
        R.logsumexp(x, out=torch.empty(4))
    with pytest.raises(RuntimeError, match="return_lse"):
        R.token_logprob(x, torch.zeros(4, dtype=torch.int64), return_lse=True)
    # the autograd variants check their inputs like the plain helpers
    with pytest.raises(ValueError, match="GPU"):
        R.logsumexp(x)
    with pytest.raises(ValueError, match="contiguous GPU"):
        R.logsumexp_dim(torch.zeros(2, 3, 4, requires_grad=True), 1)
    for call in (lambda: R.logsumexp(x, handle_=1),
                 lambda: R.logsumexp_dim(torch.zeros(2, 3, requires_grad=True), 0, handle_=1),
                 lambda: R.token_logprob(x, torch.zeros(4, dtype=torch.int64), handle_=1)):
        with pytest.raises(RuntimeError, match="handle_"):
            call()
    with torch.no_grad():  # grad mode off: the plain path and its own checks
        with pytest.raises(ValueError, match="GPU"):
            R.logsumexp(x, out=torch.empty(4))
