import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_sessionstart(session):
    """Build the HIP library in-tree when it is not there yet (a fresh checkout
    on a machine with hipcc); a library that is already built is used as is.
    The float64 oracle builds itself on first use the same way."""
    import shutil
    have_hipcc = shutil.which("hipcc") or Path("/opt/rocm/bin/hipcc").exists()
    pkg = ROOT / "row_wise_log_amd"
    if have_hipcc and not (pkg / "liblse_amd.so").exists():
        from row_wise_log_amd import build
        build.build()
    if have_hipcc and not (pkg / "libread_control.so").exists():
        from row_wise_log_amd import build
        build.build_control()


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    return _oracle.default()
