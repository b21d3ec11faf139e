"""bench.py's host-side tools, on the CPU: the rocprofv3 CSV summaries, the
traffic record they write, the source hash it is tied to, and the plan
syntax of the A/B mode. Synthetic CSV files stand in for a profiler run.
"""
import csv
import re

import pytest

import bench

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
                "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
                "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
                "Counter_Value", "Start_Timestamp", "End_Timestamp"]
HEADLINE = ("void lse::stream_rows<(lse::DType)1, 512, 4, false, false>(char const*, long, long, "
            "float*, int, unsigned int*, unsigned int*, long const*, float*)")


def write_csv(path, cols, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, 0) for c in cols})


def test_short_kernel_name():
    assert bench.short_kernel_name(HEADLINE) == \
        "void lse::stream_rows<(lse::DType)1, 512, 4, false, false>"
    assert bench.short_kernel_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_trace_summary_and_runs(tmp_path):
    rows, t, did = [], 0, 0
    # 60 headline launches of 20 us, 5 of another kernel, 60 more of 22 us
    for n, name, dur in ((60, HEADLINE, 20_000), (5, "other_kernel(int)", 1_000),
                         (60, HEADLINE, 22_000)):
        for _ in range(n):
            did += 1
            rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Start_Timestamp": t,
                         "End_Timestamp": t + dur, "Workgroup_Size_X": 512,
                         "Grid_Size_X": 512 * 512})
            t += dur + 100
    write_csv(tmp_path / "host" / "1" / "run_kernel_trace.csv", TRACE_COLS, rows)
    table = bench.summarize_trace(str(tmp_path))
    line = next(l for l in table.splitlines() if "stream_rows" in l)
    assert "| 512 x 512 | 120 | 21.00 |" in line
    runs = bench.summarize_trace_runs(str(tmp_path)).splitlines()
    assert sum("stream_rows" in l for l in runs) == 2     # two runs of 60, the 5 in between dropped
    assert "| 1 |" in runs[2] and "20.00" in runs[2] and "| 66 |" in runs[3] and "22.00" in runs[3]


def counter_rows(kernel, counter, values, start_id):
    return [{"Dispatch_Id": start_id + i, "Kernel_Name": kernel, "Counter_Name": counter,
             "Counter_Value": v} for i, v in enumerate(values)]


def test_traffic_record_from_counter_runs(tmp_path, monkeypatch):
    """Calibration on the first three copy dispatches only; every workload's
    kernel found by the name its plan launches; bytes = KiB x 1024 x factor."""
    from row_wise_log_amd import binding as B
    import workloads
    names = {}
    for cfg in (1, 2, 3, 4, 5):
        sp = workloads.SPECS[cfg]
        plan = B.lse_plan(bench.dtype_code_of(B, sp.dtype), sp.rows, sp.cols, sp.cols, 0, 256, 0)
        names[cfg] = bench.plan_kernel_name(plan, sp.dtype, sp.cols) + "(char const*)"
    copy_kib = (256 << 20) / 1024
    for counter, factor in (("FETCH_SIZE", 2.0), ("WRITE_SIZE", 1.0)):
        rows = counter_rows("__amd_rocclr_copyBuffer", counter, [copy_kib / factor] * 3, 1)
        rows += counter_rows("__amd_rocclr_copyBuffer", counter, [5.0] * 8, 100)  # later copies
        did = 1000
        for cfg, name in names.items():
            sp = workloads.SPECS[cfg]
            esize = 4 if sp.dtype == "f32" else 2
            kib = (sp.rows * sp.cols * esize if counter == "FETCH_SIZE" else 4 * sp.rows) / 1024
            rows += counter_rows(name, counter, [kib / factor] * 4, did)
            did += 10
        write_csv(tmp_path / counter / "run_counter_collection.csv", COUNTER_COLS, rows)
    text = bench.write_traffic(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"),
                               256 << 20, "rocprofv3 --pmc COUNTER -- python3 bench.py")
    assert f"kernel_source_hash: {bench.kernel_source_hash()}" in text
    for cfg in (1, 2, 3, 4, 5):
        sp = workloads.SPECS[cfg]
        esize = 4 if sp.dtype == "f32" else 2
        got = float(re.search(rf"config{cfg}_bytes_per_launch: (\d+)", text).group(1))
        assert got == pytest.approx(sp.rows * sp.cols * esize + 4 * sp.rows, rel=1e-9)
        assert "traffic/algorithmic = 1.0000" in text.split(f"# config {cfg}:")[1].splitlines()[0]


def test_committed_traffic_names_the_planned_kernels():
    """profiles/traffic.txt lists, per workload, the kernel the planner picks."""
    from row_wise_log_amd import binding as B
    import workloads
    text = bench.TRAFFIC_FILE.read_text()
    for cfg in (1, 2, 3, 4, 5):
        sp = workloads.SPECS[cfg]
        plan = B.lse_plan(bench.dtype_code_of(B, sp.dtype), sp.rows, sp.cols, sp.cols, 0, 256, 0)
        assert f"# config {cfg}: {bench.plan_kernel_name(plan, sp.dtype, sp.cols)}:" in text


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() {\n  return 1;  // one\n}\n/* a block\n   comment */\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [src])
    h0 = bench.kernel_source_hash()
    src.write_text("// new prose\nint f() {\n  return 1;  // another\n}\n\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f() {\n  return 2;\n}\n")
    assert bench.kernel_source_hash() != h0


def test_parse_plan():
    assert bench.parse_plan("auto")["schedule"] == "auto"
    p = bench.parse_plan("schedule=split_row,block=256,parts=4")
    assert (p["schedule"], p["block"], p["parts"], p["unroll"]) == ("split_row", 256, 4, 0)
    with pytest.raises(SystemExit):
        bench.parse_plan("blocks=256")


def test_event_passes_are_the_runs_after_a_control_lead(tmp_path):
    """An event pass is a library kernel's run whose previous run is a control
    (the lead) and whose run before that is the same kernel and shape (its
    warmup and wall-clock pass); only its first `steps` dispatches count."""
    ctl = "void (anonymous namespace)::read_chunks<512>(unsigned int const*, long, long, unsigned int*)"
    other = ("void lse::stream_rows<(lse::DType)0, 64, 4, true, false>(char const*, long, long, "
             "float*, int, unsigned int*, unsigned int*, long const*, float*)")
    rows, t, did = [], 0, 0
    # control (its own timed run), LSE warmup + wall pass, control lead, LSE event
    # pass + 60 single calls (slower), then another kernel after a control run
    # (not an event pass: no earlier run of it)
    for n, name, dur in ((100, ctl, 21_000), (300, HEADLINE, 22_000), (50, ctl, 21_000),
                         (1000, HEADLINE, 21_500), (60, HEADLINE, 30_000), (80, ctl, 5_000),
                         (1200, other, 5_000)):
        for _ in range(n):
            did += 1
            rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Start_Timestamp": t,
                         "End_Timestamp": t + dur, "Workgroup_Size_X": 512,
                         "Grid_Size_X": 512 * 512})
            t += dur + 100
    write_csv(tmp_path / "host" / "1" / "run_kernel_trace.csv", TRACE_COLS, rows)
    table = bench.summarize_event_passes(str(tmp_path), steps=1000).splitlines()
    assert len(table) == 3, table
    assert "| 451 |" in table[2] and "| 1000 | 21.50 |" in table[2] and "| 50, 21.00 |" in table[2]
    # span: 1000 dispatches of 21.5 us with 0.1 us between them
    assert "| 21.60 |" in table[2]

