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
