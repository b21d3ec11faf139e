"""The C ABI from plain C: tests/c_abi/lse_example.c includes include/lse.h,
links the in-tree library and calls it with no Python or torch in between.

* CPU: the program compiles as strict C11 (-Wall -Wextra -Werror) and links
  against liblse_amd.so, so the header is valid C and every symbol it uses
  resolves.
* GPU: the program runs as a child process and checks lse_forward on rows of
  constants (closed form c + ln N, fp32 and bf16), error returns, an empty
  row and a row of -inf.
"""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "tests" / "c_abi" / "lse_example.c"
LIBDIR = ROOT / "row_wise_log_amd"
ROCM = Path("/opt/rocm")


def build_example(out: Path) -> Path:
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not (LIBDIR / "liblse_amd.so").exists():
        pytest.fail("liblse_amd.so is not built (python -m row_wise_log_amd.build)")
    exe = out / "lse_example"
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT / 'include'}", f"-I{ROCM / 'include'}", str(SRC), "-o", str(exe),
           f"-L{LIBDIR}", "-llse_amd", f"-L{ROCM / 'lib'}", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM / 'lib'}"]
    proc = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, proc.stderr
    return exe


def test_c_program_compiles_and_links(tmp_path):
    exe = build_example(tmp_path)
    assert exe.exists()


@pytest.mark.gpu
def test_c_program_runs(tmp_path):
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() == 0:  # counts devices without initialising one
        pytest.skip("no GPU")
    exe = build_example(tmp_path)
    print("c_abi example: running", exe, flush=True)
    proc = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, f"exit {proc.returncode}: {proc.stderr}"
    assert proc.stdout.strip() == "ok"
