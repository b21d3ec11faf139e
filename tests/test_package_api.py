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
        R.logsumexp_dim(torch.zeros(2, 3, dtype=torch.float16), 1)
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
