"""The C ABI on the host: symbols, argument checks and the launch planner.

These run without a GPU. lse_forward checks its arguments before any HIP
call (handle last), so a NULL handle with one bad argument reports that
argument's error; lse_plan is the planner lse_forward uses, exported as a
pure host function.
"""
import re
import shutil
import subprocess
from pathlib import Path

import pytest

from row_wise_log_amd import binding as B

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "lse.h"
F32, BF16 = B.LSE_DTYPE_F32, B.LSE_DTYPE_BF16


@pytest.fixture(scope="module")
def lib():
    return B.load()


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|lse_status_t)\s*(lse_\w+)\s*\(",
                                 text, re.M)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert {"lse_create", "lse_forward", "lse_destroy", "lse_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", str(B.LIBRARY)], capture_output=True,
                             text=True, check=True).stdout
        exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
        assert set(names) <= exported
        assert set(B.EXPORTS) == set(names)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_is_valid_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "lse.h"\nint main(void) { lse_plan_t p; (void)p; '
                   'return (int)sizeof(lse_status_t) - 4 + (int)LSE_OK; }\n')
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROOT / 'include'}", "-I/opt/rocm/include", "-c", str(src),
                    "-o", str(tmp_path / "use.o")], check=True)


def test_status_strings(lib):
    for code, name in [(0, "LSE_OK"), (1, "LSE_ERR_INVALID_ARG"), (2, "LSE_ERR_UNSUPPORTED_DTYPE"),
                       (3, "LSE_ERR_NO_DEVICE"), (4, "LSE_ERR_ALLOC"), (5, "LSE_ERR_HIP")]:
        assert B.status_string(code) == name
    assert B.status_string(99) == "LSE_ERR_UNKNOWN"


def test_create_without_device_reports_no_device(lib):
    try:
        h = B.lse_create(0)
    except B.LseError as e:
        assert e.status == B.LSE_ERR_NO_DEVICE
    else:
        B.lse_destroy(h)
        pytest.skip("a GPU is present")
    assert B.load().lse_create(None, 0) == B.LSE_ERR_INVALID_ARG


def test_destroy_null_is_ok(lib):
    B.lse_destroy(None)


@pytest.mark.parametrize("args, status", [
    # (x, dtype, rows, cols, row_stride, out) with a NULL handle
    ((16, 7, 4, 4, 4, 16), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, -1, 4, 4, 4, 16), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, F32, -1, 4, 4, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 4, -1, 4, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 1 << 31, 4, 4, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 4, 1 << 31, 1 << 31, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 4, 8, 7, 16), B.LSE_ERR_INVALID_ARG),           # stride < cols
    ((16, F32, 4, 8, 1 << 62, 16), B.LSE_ERR_INVALID_ARG),     # byte offsets overflow
    ((18, F32, 4, 4, 4, 16), B.LSE_ERR_INVALID_ARG),           # x not 4-byte aligned
    ((17, BF16, 4, 4, 4, 16), B.LSE_ERR_INVALID_ARG),          # x not 2-byte aligned
    ((None, F32, 4, 4, 4, 16), B.LSE_ERR_INVALID_ARG),         # NULL x with work
    ((16, F32, 4, 4, 4, None), B.LSE_ERR_INVALID_ARG),         # NULL out
    ((16, F32, 4, 4, 4, 18), B.LSE_ERR_INVALID_ARG),           # out not 4-byte aligned
    ((16, F32, 4, 4, 4, 16), B.LSE_ERR_INVALID_ARG),           # all fine but the handle
    ((None, F32, 0, 4, 4, None), B.LSE_ERR_INVALID_ARG),       # rows = 0 still needs a handle
])
def test_forward_argument_checks(lib, args, status):
    x, dtype, rows, cols, stride, out = args
    assert B.lse_forward_status(None, x, dtype, rows, cols, stride, out) == status


@pytest.mark.parametrize("args, status", [
    # (x, dtype, rows, cols, row_stride, out): lse_forward_noalloc checks the
    # same arguments before any HIP call and needs no handle
    ((16, 7, 4, 4, 4, 16), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, F32, -1, 4, 4, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 4, 1 << 31, 1 << 31, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 4, 8, 7, 16), B.LSE_ERR_INVALID_ARG),           # stride < cols
    ((17, BF16, 4, 4, 4, 16), B.LSE_ERR_INVALID_ARG),          # x not 2-byte aligned
    ((None, F32, 4, 4, 4, 16), B.LSE_ERR_INVALID_ARG),         # NULL x with work
    ((16, F32, 4, 4, 4, None), B.LSE_ERR_INVALID_ARG),         # NULL out
    ((16, F32, 4, 4, 4, 18), B.LSE_ERR_INVALID_ARG),           # out not 4-byte aligned
    ((None, F32, 0, 4, 4, None), B.LSE_OK),                    # rows = 0: nothing to do
])
def test_forward_noalloc_argument_checks(lib, args, status):
    x, dtype, rows, cols, stride, out = args
    assert B.lse_forward_noalloc_status(x, dtype, rows, cols, stride, out) == status


def test_forward_noalloc_without_device_reports_no_device(lib):
    try:
        h = B.lse_create(0)
    except B.LseError:
        pass
    else:
        B.lse_destroy(h)
        pytest.skip("a GPU is present")
    assert B.lse_forward_noalloc_status(16, F32, 4, 4, 4, 16) == B.LSE_ERR_NO_DEVICE


@pytest.mark.parametrize("args, status", [
    # (x, dtype, rows, cols, row_stride, targets, logp, lse_out) with a NULL handle
    ((16, 7, 4, 4, 4, 64, 16, None), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, F32, -1, 4, 4, 64, 16, None), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 4, 8, 7, 64, 16, None), B.LSE_ERR_INVALID_ARG),      # stride < cols
    ((18, F32, 4, 4, 4, 64, 16, None), B.LSE_ERR_INVALID_ARG),      # x misaligned
    ((16, F32, 4, 4, 4, None, 16, None), B.LSE_ERR_INVALID_ARG),    # NULL targets
    ((16, F32, 4, 4, 4, 68, 16, None), B.LSE_ERR_INVALID_ARG),      # targets not 8-byte aligned
    ((16, F32, 4, 4, 4, 64, None, None), B.LSE_ERR_INVALID_ARG),    # NULL logp
    ((16, F32, 4, 4, 4, 64, 18, None), B.LSE_ERR_INVALID_ARG),      # logp misaligned
    ((16, F32, 4, 4, 4, 64, 16, 18), B.LSE_ERR_INVALID_ARG),        # lse_out misaligned
    ((16, F32, 4, 4, 4, 64, 16, 32), B.LSE_ERR_INVALID_ARG),        # all fine but the handle
    ((None, F32, 0, 4, 4, None, None, None), B.LSE_ERR_INVALID_ARG),  # rows = 0 needs a handle
])
def test_token_logprob_argument_checks(lib, args, status):
    x, dtype, rows, cols, stride, targets, logp, lse = args
    assert B.lse_token_logprob_status(None, x, dtype, rows, cols, stride, targets, logp,
                                      lse) == status


@pytest.mark.parametrize("args, status", [
    # (x, dtype, rows, cols, row_stride, lse, grad_out, grad_x, grad_row_stride), NULL handle
    ((16, 7, 4, 4, 4, 64, 64, 128, 4), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, F32, -1, 4, 4, 64, 64, 128, 4), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 4, 8, 7, 64, 64, 128, 8), B.LSE_ERR_INVALID_ARG),      # x stride < cols
    ((16, F32, 4, 8, 8, 64, 64, 128, 7), B.LSE_ERR_INVALID_ARG),      # grad stride < cols
    ((16, F32, 4, 8, 8, 64, 64, 128, 1 << 62), B.LSE_ERR_INVALID_ARG),  # grad offsets overflow
    ((16, F32, 4, 4, 4, None, 64, 128, 4), B.LSE_ERR_INVALID_ARG),    # NULL lse
    ((16, F32, 4, 4, 4, 64, None, 128, 4), B.LSE_ERR_INVALID_ARG),    # NULL grad_out
    ((16, F32, 4, 4, 4, 64, 64, None, 4), B.LSE_ERR_INVALID_ARG),     # NULL grad_x
    ((16, F32, 4, 4, 4, 66, 64, 128, 4), B.LSE_ERR_INVALID_ARG),      # lse misaligned
    ((16, F32, 4, 4, 4, 64, 66, 128, 4), B.LSE_ERR_INVALID_ARG),      # grad_out misaligned
    ((16, F32, 4, 4, 4, 64, 64, 130, 4), B.LSE_ERR_INVALID_ARG),      # fp32 grad_x misaligned
    ((16, BF16, 4, 4, 4, 64, 64, 129, 4), B.LSE_ERR_INVALID_ARG),     # bf16 grad_x misaligned
    ((16, F32, 4, 4, 4, 64, 64, 128, 4), B.LSE_ERR_INVALID_ARG),      # all fine but the handle
    ((None, F32, 0, 4, 4, None, None, None, 4), B.LSE_ERR_INVALID_ARG),  # rows = 0 needs a handle
])
def test_backward_argument_checks(lib, args, status):
    assert B.lse_backward_status(None, *args) == status


@pytest.mark.parametrize("args, status", [
    # (x, dtype, rows, cols, row_stride, targets, lse, grad_logp, grad_x, grad_row_stride)
    ((16, 7, 4, 4, 4, 256, 64, 64, 128, 4), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, F32, 4, 8, 7, 256, 64, 64, 128, 8), B.LSE_ERR_INVALID_ARG),     # x stride < cols
    ((16, F32, 4, 8, 8, 256, 64, 64, 128, 7), B.LSE_ERR_INVALID_ARG),     # grad stride < cols
    ((16, F32, 4, 4, 4, None, 64, 64, 128, 4), B.LSE_ERR_INVALID_ARG),    # NULL targets
    ((16, F32, 4, 4, 4, 260, 64, 64, 128, 4), B.LSE_ERR_INVALID_ARG),     # targets misaligned
    ((16, F32, 4, 4, 4, 256, None, 64, 128, 4), B.LSE_ERR_INVALID_ARG),   # NULL lse
    ((16, F32, 4, 4, 4, 256, 64, None, 128, 4), B.LSE_ERR_INVALID_ARG),   # NULL grad_logp
    ((16, F32, 4, 4, 4, 256, 64, 64, None, 4), B.LSE_ERR_INVALID_ARG),    # NULL grad_x
    ((16, F32, 4, 4, 4, 256, 64, 64, 128, 4), B.LSE_ERR_INVALID_ARG),     # all fine but the handle
    ((None, F32, 0, 4, 4, None, None, None, None, 4), B.LSE_ERR_INVALID_ARG),  # rows = 0
])
def test_token_logprob_backward_argument_checks(lib, args, status):
    assert B.lse_token_logprob_backward_status(None, *args) == status


@pytest.mark.parametrize("args, status", [
    # (x, dtype, outer, n, inner, out) with a NULL handle
    ((16, 7, 2, 3, 4, 16), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, F32, -1, 3, 4, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 2, -3, 4, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 2, 3, -4, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 2, 1 << 31, 4, 16), B.LSE_ERR_INVALID_ARG),       # n too large
    ((16, F32, 1 << 21, 3, 1 << 20, 16), B.LSE_ERR_INVALID_ARG),  # outer * inner > 2^40
    ((16, F32, 1 << 20, 1 << 30, 1 << 12, 16), B.LSE_ERR_INVALID_ARG),  # element count overflows
    ((18, F32, 2, 3, 4, 16), B.LSE_ERR_INVALID_ARG),             # x misaligned
    ((16, F32, 2, 3, 4, 18), B.LSE_ERR_INVALID_ARG),             # out misaligned
    ((None, F32, 2, 3, 4, 16), B.LSE_ERR_INVALID_ARG),           # NULL x with work
    ((16, F32, 2, 3, 4, None), B.LSE_ERR_INVALID_ARG),           # NULL out
    ((16, F32, 2, 3, 4, 16), B.LSE_ERR_INVALID_ARG),             # all fine but the handle
    ((None, F32, 0, 3, 4, None), B.LSE_ERR_INVALID_ARG),         # nothing to do still needs a handle
])
def test_forward_dim_argument_checks(lib, args, status):
    assert B.lse_forward_dim_status(None, *args) == status


@pytest.mark.parametrize("args, status", [
    # (x, dtype, outer, n, inner, lse, grad_out, grad_x) with a NULL handle
    ((16, 7, 2, 3, 4, 16, 16, 16), B.LSE_ERR_UNSUPPORTED_DTYPE),
    ((16, F32, -1, 3, 4, 16, 16, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 2, -3, 4, 16, 16, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 2, 3, -4, 16, 16, 16), B.LSE_ERR_INVALID_ARG),
    ((16, F32, 2, 1 << 31, 4, 16, 16, 16), B.LSE_ERR_INVALID_ARG),       # n too large
    ((16, F32, 1 << 21, 3, 1 << 20, 16, 16, 16), B.LSE_ERR_INVALID_ARG),  # outer * inner > 2^40
    ((18, F32, 2, 3, 4, 16, 16, 16), B.LSE_ERR_INVALID_ARG),             # x misaligned
    ((16, BF16, 2, 3, 4, 16, 16, 17), B.LSE_ERR_INVALID_ARG),            # grad_x misaligned
    ((16, F32, 2, 3, 4, 18, 16, 16), B.LSE_ERR_INVALID_ARG),             # lse misaligned
    ((16, F32, 2, 3, 4, 16, 18, 16), B.LSE_ERR_INVALID_ARG),             # grad_out misaligned
    ((None, F32, 2, 3, 4, 16, 16, 16), B.LSE_ERR_INVALID_ARG),           # NULL x with work
    ((16, F32, 2, 3, 4, None, 16, 16), B.LSE_ERR_INVALID_ARG),           # NULL lse
    ((16, F32, 2, 3, 4, 16, None, 16), B.LSE_ERR_INVALID_ARG),           # NULL grad_out
    ((16, F32, 2, 3, 4, 16, 16, None), B.LSE_ERR_INVALID_ARG),           # NULL grad_x
    ((16, F32, 2, 3, 4, 16, 16, 16), B.LSE_ERR_INVALID_ARG),             # all fine but the handle
    ((None, F32, 2, 0, 4, None, None, None), B.LSE_ERR_INVALID_ARG),     # nothing to do still needs a handle
])
def test_backward_dim_argument_checks(lib, args, status):
    assert B.lse_backward_dim_status(None, *args) == status


def test_forward_accepts_stride_below_cols_for_one_row(lib):
    # one row: row_stride is ignored, so only the handle is wrong
    assert B.lse_forward_status(None, 16, F32, 1, 8, 0, 16) == B.LSE_ERR_INVALID_ARG
    assert B.lse_forward_status(None, 16, BF16, 1, 8, 3, 16) == B.LSE_ERR_INVALID_ARG


def test_setters_reject_bad_values(lib):
    assert lib.lse_set_schedule(None, 1) == B.LSE_ERR_INVALID_ARG
    assert lib.lse_set_tuning(None, 0, 0, 0, 0, 0) == B.LSE_ERR_INVALID_ARG


# ---- the planner ------------------------------------------------------------

def plan(dtype, rows, cols, stride=None, addr=0, n_cu=256, schedule=0):
    return B.lse_plan(dtype, rows, cols, cols if stride is None else stride, addr, n_cu, schedule)


def test_plan_for_the_five_workloads():
    p1 = plan(F32, 64, 32000)                             # 64 rows: split, 16 parts each
    assert p1["schedule"] == B.LSE_SCHED_SPLIT_ROW and p1["grid"] == 1024 and p1["block"] == 64
    p2 = plan(BF16, 512, 128256)
    assert p2["schedule"] == B.LSE_SCHED_ROW_PER_WG and p2["grid"] == 512
    assert (p2["block"], p2["unroll"]) == (512, 4)        # two rows per CU
    p3 = plan(BF16, 4096, 262144)
    assert p3["schedule"] == B.LSE_SCHED_ROW_PER_WG and p3["grid"] == 4096
    p4 = plan(F32, 65536, 4096)
    assert p4["schedule"] == B.LSE_SCHED_ROW_PER_WG and (p4["block"], p4["unroll"]) == (256, 4)
    p5 = plan(F32, 1 << 24, 16)
    assert p5["schedule"] == B.LSE_SCHED_ROWS_PER_WAVE
    assert (p5["lanes_per_row"], p5["loads_per_lane"], p5["rows_per_wave"]) == (4, 1, 64)
    assert p5["grid"] == 256 * 8 // 4                    # 8 wavefronts per CU, 4 per block


def test_plan_rows_zero():
    assert plan(F32, 0, 100)["schedule"] == 0 and plan(F32, 0, 100)["grid"] == 0


def regs_instance(g, vpl, vec):
    """The register-rows kernel instances that exist (lse_kernels.hip)."""
    if vpl == 1:
        return True
    if vpl in (2, 4):
        return g <= 4 or g == 64
    return not vec and g == 64 and vpl in (8, 16)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_plan_register_rows_cover_every_element(dtype):
    k = 4 if dtype == F32 else 8
    esize = 16 // k
    for cols in list(range(0, 80)) + [127, 128, 129, 255, 256, 257, 1023, 1024, 1025, 2047,
                                      2048, 2049, 4095, 4096, 4097]:
        for stride_pad, addr in [(0, 0), (k, 0), (1, 0), (0, 4 if dtype == F32 else 2)]:
            stride = cols + stride_pad
            p = plan(dtype, 100, cols, stride, addr)
            aligned = addr % 16 == 0 and (stride * esize) % 16 == 0
            if cols == 0 or (aligned and 1 <= cols // k <= 256) or \
                    ((not aligned or cols < k) and cols <= 1024):
                assert p["schedule"] == B.LSE_SCHED_ROWS_PER_WAVE, (cols, stride, addr)
            else:
                assert p["schedule"] != B.LSE_SCHED_ROWS_PER_WAVE, (cols, stride, addr)
                continue
            g, vpl = p["lanes_per_row"], p["loads_per_lane"]
            assert g in (1, 2, 4, 8, 16, 32, 64)
            assert regs_instance(g, vpl, p["vector_loads"] == 1), (cols, g, vpl)
            if p["vector_loads"]:
                assert aligned
                assert g * vpl >= cols // k and g >= cols % k and cols // k >= 1
            else:
                assert g * vpl >= cols
            assert p["rows_per_wave"] == (64 // g) * (4 if vpl == 1 else 2 if vpl == 2 else 1)


def test_plan_streaming_block_follows_row_length():
    # about 32 fp32 or 64 bf16 elements per lane, 64..256 threads
    assert plan(F32, 100000, 2048)["block"] == 128      # 8 KiB rows
    assert plan(F32, 100000, 4096)["block"] == 256      # 16 KiB rows
    assert plan(F32, 100000, 1 << 16)["block"] == 256
    assert plan(BF16, 100000, 4096)["block"] == 64      # 8 KiB rows
    assert plan(BF16, 100000, 8192)["block"] == 128
    assert plan(F32, 200, 1 << 16)["block"] == 512      # fewer rows than CUs
    assert plan(F32, 100, 1 << 14)["block"] == 512      # 64 KiB rows are not split
    assert plan(F32, 223, 1 << 16)["block"] == 512
    assert plan(F32, 224, 1 << 16)["block"] == 256      # one or two rows per CU
    assert plan(F32, 479, 1 << 16)["block"] == 256
    assert plan(F32, 480, 1 << 16)["block"] == 512      # (nearly) two rows on every CU
    assert plan(F32, 512, 1 << 16)["block"] == 512
    assert plan(F32, 513, 1 << 16)["block"] == 256


def test_plan_long_rows_and_few_rows():
    # At most half as many rows as CUs (under 256 KiB: fewer than 3/8),
    # longer than 64 KiB: split, with the
    # wavefronts for one batch (4 vectors) per lane, at most the row's share of
    # 4 per CU; up to 64 parts of 64 threads, then wider workgroups.
    p = plan(F32, 8, 1 << 20)             # 4 MiB rows: share 128 wavefronts each
    assert p["schedule"] == B.LSE_SCHED_SPLIT_ROW and p["parts"] == 64 and p["block"] == 128
    assert p["grid"] == 512 and p["workspace_bytes"] == 8 * 64 * 8 + 8 * 4
    p = plan(BF16, 1, 128256)             # one vocabulary row: 64 one-batch parts
    assert (p["schedule"], p["parts"], p["block"], p["grid"]) == (B.LSE_SCHED_SPLIT_ROW, 64, 64, 64)
    p = plan(BF16, 32, 128256)            # share 32 wavefronts per row
    assert (p["parts"], p["block"], p["grid"]) == (32, 64, 1024)
    # the share rounds up to a power of two: 40 rows -> 26 -> 32, 75 -> 14 -> 16
    assert (plan(BF16, 40, 1810534)["parts"], plan(BF16, 40, 1810534)["block"]) == (32, 64)
    assert (plan(BF16, 75, 383639)["parts"], plan(BF16, 75, 383639)["block"]) == (16, 64)
    assert plan(F32, 3, 292775)["parts"] == 64 and plan(F32, 3, 292775)["block"] == 512
    p = plan(F32, 64, 32000)              # 125 KiB rows, share 16
    assert (p["schedule"], p["parts"], p["block"]) == (B.LSE_SCHED_SPLIT_ROW, 16, 64)
    p = plan(F32, 1, 1 << 28)
    assert p["parts"] == B.LSE_SPLIT_MAX_PARTS and p["block"] == 512
    assert plan(F32, 128, 1 << 16)["schedule"] == B.LSE_SCHED_SPLIT_ROW
    assert plan(F32, 128, 1 << 16)["parts"] == 8
    assert plan(F32, 129, 1 << 16)["schedule"] == B.LSE_SCHED_ROW_PER_WG
    assert plan(F32, 129, 1 << 16)["block"] == 512
    assert plan(F32, 8, (1 << 14) + 4)["schedule"] == B.LSE_SCHED_SPLIT_ROW
    assert plan(F32, 8, 1 << 14)["schedule"] == B.LSE_SCHED_ROW_PER_WG   # 64 KiB rows
    assert plan(F32, 95, 1 << 15)["schedule"] == B.LSE_SCHED_SPLIT_ROW   # 128 KiB rows: 3/8
    assert plan(F32, 96, 1 << 15)["schedule"] == B.LSE_SCHED_ROW_PER_WG
    assert plan(F32, 96, 1 << 16)["schedule"] == B.LSE_SCHED_SPLIT_ROW   # 256 KiB rows: 1/2
    # just over one row per CU (up to 5/4), rows of 1 MiB and more: quarters of 256 threads
    p = plan(F32, 257, 1 << 18)
    assert (p["schedule"], p["parts"], p["block"]) == (B.LSE_SCHED_SPLIT_ROW, 4, 256)
    assert plan(F32, 320, 1 << 18)["parts"] == 4
    assert plan(F32, 321, 1 << 18)["schedule"] == B.LSE_SCHED_ROW_PER_WG
    assert plan(F32, 256, 1 << 18)["schedule"] == B.LSE_SCHED_ROW_PER_WG
    assert plan(F32, 300, (1 << 18) - 4)["schedule"] == B.LSE_SCHED_ROW_PER_WG   # under 1 MiB
    # the quarters belong to the automatic choice only: a forced split in the
    # same band of rows keeps the general rule (the rows' share of 4 wavefronts
    # per CU: 4 parts of 64 threads), for short rows and long ones alike
    p = plan(F32, 300, 1 << 14, schedule=3)
    assert (p["schedule"], p["parts"], p["block"]) == (B.LSE_SCHED_SPLIT_ROW, 4, 64)
    p = plan(F32, 300, 1 << 18, schedule=3)
    assert (p["schedule"], p["parts"], p["block"]) == (B.LSE_SCHED_SPLIT_ROW, 4, 64)
    # unaligned long rows stream with a head peel
    assert plan(BF16, 4, 5001, 5001)["schedule"] == B.LSE_SCHED_ROW_PER_WG
    assert plan(BF16, 4, 500001, 500001)["schedule"] == B.LSE_SCHED_SPLIT_ROW
    assert plan(BF16, 4000, 500001, 500001)["schedule"] == B.LSE_SCHED_ROW_PER_WG


def test_plan_forced_schedules():
    assert plan(F32, 1 << 24, 16, schedule=2)["schedule"] == B.LSE_SCHED_ROW_PER_WG
    p = plan(F32, 1 << 24, 16, schedule=3)
    assert p["schedule"] == B.LSE_SCHED_SPLIT_ROW and p["grid"] == B.LSE_SPLIT_MAX_ROWS * 2
    # rows longer than registers hold cannot stay on ROWS_PER_WAVE
    assert plan(F32, 4, 1 << 20, schedule=1)["schedule"] == B.LSE_SCHED_ROW_PER_WG
    assert plan(F32, 4, 1024, 1025, schedule=1)["schedule"] == B.LSE_SCHED_ROWS_PER_WAVE


def test_plan_rejects_bad_args():
    with pytest.raises(B.LseError):
        B.lse_plan(F32, 4, 8, 8, 0, 0, 0)
    with pytest.raises(B.LseError):
        B.lse_plan(F32, 4, 8, 8, 0, 256, 9)
    with pytest.raises(B.LseError):
        B.lse_plan(5, 4, 8, 8, 0, 256, 0)


# --- planner invariants over random shapes (hypothesis) -------------------

from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402


def _log_int(lo, hi):
    """Integers spread over magnitudes, with the edges of each power of two."""
    return st.one_of(st.integers(lo, min(hi, 64)),
                     st.builds(lambda e, d: max(lo, min(hi, (1 << e) + d)),
                               st.integers(0, hi.bit_length()), st.integers(-2, 2)))


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(dtype=st.sampled_from([F32, BF16]), rows=_log_int(1, 1 << 24), cols=_log_int(0, 1 << 26),
       pad=st.sampled_from([0, 1, 3, 8, 64]), mis=st.integers(0, 7),
       n_cu=st.sampled_from([1, 32, 104, 256, 304]), schedule=st.sampled_from([0, 1, 2, 3]))
def test_plan_invariants(dtype, rows, cols, pad, mis, n_cu, schedule):
    """Whatever the shape, the plan is one the kernels can run: an existing
    instance, every element covered, grids and workspace within their limits."""
    k = 4 if dtype == F32 else 8
    esize = 16 // k
    stride = cols + pad
    addr = (mis * esize) % 16
    p = B.lse_plan(dtype, rows, cols, stride, addr, n_cu, schedule)
    aligned = addr % 16 == 0 and (rows == 1 or (stride * esize) % 16 == 0)
    assert p["schedule"] in (B.LSE_SCHED_ROWS_PER_WAVE, B.LSE_SCHED_ROW_PER_WG,
                             B.LSE_SCHED_SPLIT_ROW)
    assert p["block"] in (64, 128, 256, 512, 1024)
    assert 1 <= p["grid"] < (1 << 31)
    if cols == 0:
        assert p["schedule"] == B.LSE_SCHED_ROWS_PER_WAVE
    if p["schedule"] == B.LSE_SCHED_ROWS_PER_WAVE:
        g, vpl = p["lanes_per_row"], p["loads_per_lane"]
        assert g in (1, 2, 4, 8, 16, 32, 64)
        assert regs_instance(g, vpl, p["vector_loads"] == 1), (g, vpl)
        if p["vector_loads"]:
            assert aligned and cols // k >= 1
            assert g * vpl >= cols // k and g >= cols % k and cols // k <= 256
        else:
            assert cols <= 1024 and g * vpl >= cols
        rounds = 4 if vpl == 1 else 2 if vpl == 2 else 1
        assert p["rows_per_wave"] == (64 // g) * rounds
        waves = -(-rows // p["rows_per_wave"])
        assert p["grid"] == -(-min(waves, n_cu * (8 if g <= 4 else 16)) // 4)
    elif p["schedule"] == B.LSE_SCHED_ROW_PER_WG:
        assert p["grid"] == rows and p["unroll"] in (4, 8) and p["vector_loads"] == 1
        few = 2 * rows <= n_cu if cols * esize >= (256 << 10) else 8 * rows < 3 * n_cu
        quarters = n_cu < rows <= 5 * n_cu // 4 and cols * esize >= (1 << 20)
        assert schedule == B.LSE_SCHED_ROW_PER_WG or not (schedule == 0 and (quarters or (
            few and cols * esize > (64 << 10))))
    else:
        batch = min(rows, B.LSE_SPLIT_MAX_ROWS)
        assert 2 <= p["parts"] <= B.LSE_SPLIT_MAX_PARTS
        assert p["parts"] <= p["block"]  # the last part merges the pairs one per thread
        assert p["grid"] == batch * p["parts"] and p["unroll"] in (4, 8)
        assert p["workspace_bytes"] == batch * p["parts"] * 8 + batch * 4
    if schedule == B.LSE_SCHED_SPLIT_ROW and cols > 0:
        assert p["schedule"] == B.LSE_SCHED_SPLIT_ROW
    if schedule == B.LSE_SCHED_ROW_PER_WG and cols > 0:
        assert p["schedule"] == B.LSE_SCHED_ROW_PER_WG
