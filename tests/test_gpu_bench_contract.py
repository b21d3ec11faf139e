"""bench.py's output contract, on the GPU: the one JSON line a run prints
carries the keys and value types a caller of the benchmark reads (metric,
value, unit, n_gpus, steps, warmup, ms_per_step, higher_is_better, scaling,
vs_baseline, dtype, data, config.workload, and the roofline and cpu_baseline
objects), with values that agree with each other. Short runs of the small
workload keep this quick; the numbers themselves are measured elsewhere.
"""
import json
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parent.parent


def run_bench(*args: str) -> dict:
    print(f"bench.py {' '.join(args)}", flush=True)
    proc = subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True,
                          text=True, timeout=280, cwd=ROOT)
    assert proc.returncode == 0, proc.stderr[-2000:]
    lines = [l for l in proc.stdout.strip().splitlines() if l.startswith("{")]
    assert len(lines) == 1, proc.stdout
    return json.loads(lines[0])


def check_common(d: dict, steps: int) -> None:
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                     ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], typ), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] >= 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["data"] == "synthetic"
    assert d["vs_baseline"] is None
    assert d["unit"] == "GB/s" and d["value"] > 0
    assert isinstance(d["config"]["workload"], str) and d["config"]["workload"]
    # value is input bytes over the wall time per step
    # (ms_per_step and launch_us_mean are printed rounded: 5e-3 relative covers a 5 us step)
    assert d["value"] == pytest.approx(d["config"]["input_bytes"] / (d["ms_per_step"] * 1e-3) / 1e9,
                                       rel=5e-3)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] and r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    # achieved is the algorithmic bytes over the event-timed mean launch
    assert r["achieved"] == pytest.approx(
        r["algorithmic_bytes_per_launch"] / (r["launch_us_mean"] * 1e-6) / 1e9, rel=5e-3)
    assert r["traffic"] is None or r["traffic"] > 0


def test_default_workload_line():
    """The headline workload (bf16 [512, 128256]) with a short timed region,
    the float64 oracle's baseline included, and the other four workloads,
    each checked on every row against the oracle."""
    d = run_bench("--steps", "20", "--warmup", "5", "--cpu-seconds", "1")
    check_common(d, 20)
    assert d["config"]["rows"] == 512 and d["config"]["cols"] == 128256
    assert d["config"]["input_dtype"] == "bf16" and d["dtype"] == "f32"
    assert len(d["config"]["input_sha256"]) == 64
    assert {"numpy", "torch", "hip", "rocm"} <= set(d["versions"])
    assert d["max_err_over_tol"] <= 1.0 and d["nonfinite_exact"] is True
    assert d["rows_checked"] == 512
    ctl = d["roofline"]["read_control"]
    assert ctl["launch_us_mean"] > 0 and 0 < ctl["frac_of_read_control"] < 2
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert isinstance(cb["sample"], str) and cb["sample"]
    # microseconds per call on few rows of the same input, with their plans
    small = d["small_shapes"]
    assert set(small) == {"bf16 [1, 128256]", "bf16 [8, 128256]", "bf16 [32, 128256]"}
    for rec in small.values():
        assert 0 < rec["us_per_call"] < 1000 and rec["plan"].startswith("split_row")
        assert rec["max_err_over_tol"] <= 1.0
    ctx = d["torch_context"]
    assert ctx["torch.logsumexp_us"] > 0 and ctx["torch.sum_us"] > 0
    # the other four workloads, every row checked
    assert set(d["configs"]) == {"1", "3", "4", "5"}
    sizes = {"1": (64, 32000), "3": (4096, 262144), "4": (65536, 4096), "5": (1 << 24, 16)}
    for k, rec in d["configs"].items():
        assert (rec["rows"], rec["cols"]) == sizes[k]
        assert rec["rows_checked"] == rec["rows"]
        assert rec["max_err_over_tol"] <= 1.0 and rec["nonfinite_exact"] is True
        assert rec["us_per_launch"] > 0 and rec["read_control"]["launch_us_mean"] > 0
        assert rec["frac_of_hbm_peak"] == pytest.approx(
            rec["algorithmic_bytes_per_launch"] / (rec["us_per_launch"] * 1e-6) / 8e12, rel=5e-3)
    rb = d["reduced_bit"]
    for k in ("f32", "bf16", "f16"):
        assert rb[k]["us_per_launch"] > 0 and rb[k]["max_err_over_tol_own_bits"] <= 1.0
    assert rb["f32"]["mae_vs_f64_of_fp32_values"] < 1e-5 < rb["f16"]["mae_vs_f64_of_fp32_values"]
    assert rb["f16"]["mae_vs_f64_of_fp32_values"] < rb["bf16"]["mae_vs_f64_of_fp32_values"]
    rw = d["configs"]["5"]["read_write_control"]
    assert rw["launch_us_mean"] > 0 and 0 < rw["frac_of_control"] < 2
    assert d["configs"]["5"]["read_control_same_geometry"]["launch_us_mean"] > 0


@pytest.mark.parametrize("args", [["--config", "1", "--graph"], ["--config", "1", "--op", "backward"],
                                  ["--config", "1", "--op", "logprob"], ["--config", "1", "--op", "dim"]])
def test_other_modes(args):
    d = run_bench(*args, "--steps", "30", "--warmup", "5", "--no-cpu-baseline", "--only")
    check_common(d, 30)
    assert d["cpu_baseline"] is None
    r = d["roofline"]
    if "backward" in args:
        assert r["copy_control"]["launch_us_mean"] > 0
    else:
        assert r["read_control"]["launch_us_mean"] > 0
    if "--graph" in args:
        assert d["config"]["timed_as"].startswith("one HIP graph")


def test_all_workloads_for_another_op():
    """--all for the token log-probability: the other four workloads under
    `configs`, each checked against the oracle on every row."""
    d = run_bench("--config", "1", "--op", "logprob", "--all", "--steps", "10", "--warmup", "2",
                  "--no-cpu-baseline")
    check_common(d, 10)
    assert set(d["configs"]) == {"2", "3", "4", "5"}
    for rec in d["configs"].values():
        assert rec["op"] == "logprob" and rec["us_per_launch"] > 0
        assert rec["rows_checked"] == rec["rows"] and rec["max_err_over_tol"] <= 1.0
