"""Host-side checks of bench.py: the one-GPU contract, the planner leg (host
only), and the algorithmic byte counts it prices the kernels with."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and r.stdout == ""


def test_rank_outside_the_workload_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--rank", "128"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "--rank 128 outside [0, 128)" in r.stderr and r.stdout == ""


def test_summarize_trace_prices_the_named_rank(tmp_path):
    """--rank 36 (LLaMA: 819 rows of 8,192 elements a bucket, 234 blocks on
    the default rank): the launch is priced with that rank's blocks."""
    import bench
    step = "void ve::(anonymous namespace)::k_step_rows<1024, 8, 4>(ve::StepArgs, unsigned int, unsigned int)"
    rows = [_trace_row(step, 0, 1000, 256 * 1024), _trace_row(step, 2000, 1200, 256 * 1024)]
    _write_csv(str(tmp_path / "kt" / "run_kernel_trace.csv"), rows)
    _write_csv(str(tmp_path / "kt" / "run_kernel_stats.csv"),
               [{"Name": step, "Calls": 2, "AverageNs": 1100000, "MinNs": 1000000, "MaxNs": 1200000}])
    out = tmp_path / "s.txt"
    _summarize("trace", "--workload", "llama", "--rank", "36", "--trace-dir", str(tmp_path / "kt"), "--command",
               "cmd", "--out", str(out))
    alg36, _, nv, nb, _ = bench._workload_alg("llama", rank=36)
    assert nb == 819 and alg36 != bench._workload_alg("llama")[0]
    txt = out.read_text()
    assert "llama rank 36 workload" in txt
    assert f"{alg36 / 1100.0 / 1e3:.1f} GB/s" in txt


def test_counter_summary_refuses_another_rank(tmp_path):
    """bench.py reads the committed HBM counters back for the default rank
    only, so they are never summarised for another one."""
    import pytest
    with pytest.raises(SystemExit, match="default rank only"):
        _summarize("counters", "--workload", "llama", "--rank", "36", "--fetch-dir", str(tmp_path),
                   "--write-dir", str(tmp_path))


def test_planner_leg_reports_padding_at_or_above_its_bound():
    import bench
    import ragged_shard_optimizer_amd as ve
    out = bench.time_planner(ve, sizes=(64, 1024))
    assert len(out) == 2 * 2 * 2  # two models, two granularities, two FSDP sizes
    for key, v in out.items():
        assert 0.0 <= v["per_layer_lower_bound_pct"] <= v["per_layer_padding_pct"] < 100.0, key
        assert 0.0 <= v["grouped_padding_pct"] < 3.0, key
        assert v["grouped_buckets"] <= v["layer_buckets"]
        assert v["per_layer_seconds"] < 5.0 and v["grouped_seconds"] < 5.0, key


def test_group_op_byte_counts():
    # zero writes the bucket (2 B per element); scale reads and writes it;
    # accumulate also reads the gradient; padding is written only
    import bench
    assert bench.GROUP_BYTES == {"zero": 2, "scale": 4, "accumulate": 6}
    assert bench.GROUP_PAD_BYTES == 2


def test_step_byte_count_matches_the_streams():
    # per valid element: bf16 gradient read + copy, fp32 master read + write,
    # two int8 codes read + write, bf16 parameter write; per block two fp32
    # scales read + written; per padding element two bf16 zeros written
    import bench
    per_elem = 2 + 2 + 4 + 4 + 2 * (1 + 1) + 2
    assert (bench.BYTES_PER_ELEM, bench.BYTES_PER_BLOCK, bench.BYTES_PER_PAD) == (per_elem, 2 * (4 + 4), 2 + 2)


# ---------------------------------------------------------------------------
# the rocprofv3 summarisers, on small synthetic CSV files of rocprofv3's layout
def _write_csv(path, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def _trace_row(name, start_us, dur_us, grid):
    return {"Kernel_Name": name, "Start_Timestamp": int(start_us * 1000), "End_Timestamp": int((start_us + dur_us) * 1000),
            "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1}


def _summarize(*argv):
    import bench
    ap_args = ["bench.py", "--summarize", *argv]
    old = sys.argv
    sys.argv = ap_args
    try:
        bench.main()
    finally:
        sys.argv = old


def test_summarize_trace_averages_the_all_bucket_step_launches(tmp_path):
    import bench
    step = "void ve::(anonymous namespace)::k_step_wg<512, 16>(ve::StepArgs)"
    rows = [_trace_row(step, 0, 1000, 234 * 512 * 80), _trace_row(step, 2000, 1200, 234 * 512 * 80),
            _trace_row(step, 4000, 50, 234 * 512)]  # a one-bucket launch (smaller grid) is left out
    _write_csv(str(tmp_path / "kt" / "run_kernel_trace.csv"), rows)
    _write_csv(str(tmp_path / "kt" / "run_kernel_stats.csv"),
               [{"Name": step, "Calls": 3, "AverageNs": 750000, "MinNs": 50000, "MaxNs": 1200000}])
    out = tmp_path / "s.txt"
    _summarize("trace", "--workload", "llama", "--trace-dir", str(tmp_path / "kt"), "--command", "cmd",
               "--out", str(out))
    alg = bench._workload_alg("llama")[0]
    txt = out.read_text()
    assert "average 1100.0 us over 2 dispatches" in txt
    assert f"{alg / 1100.0 / 1e3:.1f} GB/s" in txt


def test_summarize_trace_picks_the_persistent_step_kernel_by_time(tmp_path):
    """A persistent step kernel's grid is one workgroup per CU whatever the
    work; a short small-block launch of the same step has a larger grid.
    The step kernel is the one with the most time."""
    dyn = "void ve::(anonymous namespace)::k_step_dyn<16>(ve::StepArgs, unsigned int, unsigned int)"
    small = "void ve::(anonymous namespace)::k_step_small<true>(ve::StepArgs)"
    rows = []
    for i in range(3):
        rows.append(_trace_row(dyn, 3000 * i, 1600 + 100 * i, 256 * 512))
        rows.append(_trace_row(small, 3000 * i + 2000, 8, 4096 * 256))
    _write_csv(str(tmp_path / "kt" / "run_kernel_trace.csv"), rows)
    _write_csv(str(tmp_path / "kt" / "run_kernel_stats.csv"),
               [{"Name": dyn, "Calls": 3, "AverageNs": 1700000, "MinNs": 1600000, "MaxNs": 1800000},
                {"Name": small, "Calls": 3, "AverageNs": 8000, "MinNs": 8000, "MaxNs": 8000}])
    out = tmp_path / "s.txt"
    _summarize("trace", "--workload", "llama", "--trace-dir", str(tmp_path / "kt"), "--command", "cmd",
               "--out", str(out))
    txt = out.read_text()
    assert "step: " + dyn in txt
    assert "average 1700.0 us over 3 dispatches" in txt
    # the warm-up dispatches can be left out (bench.py's --warmup)
    _summarize("trace", "--workload", "llama", "--trace-dir", str(tmp_path / "kt"), "--command", "cmd",
               "--out", str(out), "--skip-first", "1")
    assert "average 1750.0 us over 2 dispatches (the first 1" in out.read_text()


def test_summarize_counters_calibrates_against_the_streaming_copy(tmp_path):
    import json
    import bench
    step = "void ve::(anonymous namespace)::k_step_wg<512, 16>(ve::StepArgs)"
    copy = "ve::(anonymous namespace)::k_stream_copy(unsigned int __vector(4) const*, unsigned int __vector(4)*, long)"
    grid = 234 * 512 * 80

    def rows(counter, copy_kib, step_kib):
        return [{"Kernel_Name": copy, "Counter_Name": counter, "Counter_Value": copy_kib, "Grid_Size": 1024 * 4096},
                {"Kernel_Name": step, "Counter_Name": counter, "Counter_Value": step_kib, "Grid_Size": grid},
                {"Kernel_Name": step, "Counter_Name": counter, "Counter_Value": step_kib, "Grid_Size": grid}]
    # the copy of 1 GiB reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), rows("FETCH_SIZE", 524288, 2097152))
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), rows("WRITE_SIZE", 1048576, 5242880))
    _summarize("counters", "--workload", "llama", "--fetch-dir", str(tmp_path / "f"), "--write-dir",
               str(tmp_path / "w"), "--copy-gib", "1", "--profiles-dir", str(tmp_path))
    d = json.load(open(tmp_path / "shard_step_llama_traffic.json"))
    assert d["fetch_factor"] == 2.0 and d["write_factor"] == 1.0
    assert d["read_bytes"] == 2097152 * 2 * 1024 and d["write_bytes"] == 5242880 * 1024
    assert d["alg_bytes_per_launch"] == bench._workload_alg("llama")[0]
    assert d["kernel_source_hash"] == bench.kernel_source_hash(bench.STEP_SOURCES)


def test_summarize_muon_per_call_times(tmp_path):
    import bench
    dma = "void ve::(anonymous namespace)::k_gemm_nt_dma<DmaCfg<128, 64, 64, 3, true>, false, true, false>(ve::GemmArgs)"
    t, rows = 0.0, []

    def call(norm_grid, gemm_us):
        nonlocal t
        for name, dur, grid in (("k_sumsq(unsigned short const*, long, double*)", 100, 262144),
                                ("k_norm_scale(double const*, int, float, float*)", 5, 256),
                                ("k_normalize_v(unsigned short const*)", 200, norm_grid),
                                (dma, gemm_us, 1000), (dma, gemm_us, 1000)):
            rows.append(_trace_row(name, t, dur, grid))
            t += dur + 1
    for _ in range(3):
        call(14680064, 1000)      # the 8192 x 28672 matrix: a warm-up call, then two timed
    rows.append(_trace_row("void at::native::other_kernel()", t, 10, 64))
    t += 20
    for us in (50, 30, 40):
        call(917504, us)          # the 2048 x 7168 matrix
    _write_csv(str(tmp_path / "kt" / "run_kernel_trace.csv"), rows)
    out = tmp_path / "m.txt"
    _summarize("muon", "--trace-dir", str(tmp_path / "kt"), "--command", "cmd", "--out", str(out))
    txt = out.read_text()
    big, small = 305 + 2000, 305 + 70        # per timed call, the warm-up left out
    assert f"8192 x 28672 (LLaMA-3-70B MLP), 5 steps: 2 timed calls, kernel time per call {big:.1f} us" in txt
    assert f"-> {bench.ns_flops(8192, 28672) / big / 1e6:.1f} TFLOP/s" in txt
    assert f"2048 x 7168 (DeepSeek-V3 routed expert), 5 steps: 2 timed calls, kernel time per call {small:.1f} us" in txt


def test_source_hash_ignores_comments_and_layout():
    import bench
    code = 'int f(int x) {\n  return x + 1;  // one more\n}\nconst char* s = "// kept";\n'
    a = bench.strip_comments(code)
    assert a == bench.strip_comments("/* a\n block */ int f(int x) { return x + 1; }\n  const char* s = \"// kept\";")
    assert '"// kept"' in a and "one more" not in a
    assert a != bench.strip_comments(code.replace("x + 1", "x + 2"))
    assert bench.strip_comments("char c = '\\''; // q") == "char c = '\\'';"
