"""Host-side pieces of bench.py: the overlap figures it reports from the
kernels' activity records, the committed traffic summary it reads, and its
refusal of more than one GPU.  No GPU needed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_union_merges_overlapping_and_touching_intervals():
    assert bench._union([(5, 7), (0, 2), (1, 3), (3, 4), (10, 12)]) == [[0, 4], [5, 7], [10, 12]]
    assert bench._union([]) == []


def test_overlap_of_hand_worked_records():
    # records: (kind, chunk, start_us, end_us); kind 0 matmul, 1 reduce, 2 gather
    recs = [(0, 0, 0.0, 100.0), (0, 0, 10.0, 110.0),      # matmul span [0, 110]
            (1, 0, 50.0, 80.0), (1, 1, 70.0, 90.0),       # reduce: union [50, 90], inside the span
            (2, 0, 105.0, 130.0)]                         # gather: [105, 130], 5 us inside
    o = bench.overlap_of(recs, comm_bytes=65e3)
    assert o["matmul_span_us"] == 110.0
    assert o["comm_active_us"] == 65.0                    # 40 + 25
    assert o["comm_hidden_us"] == 45.0                    # 40 + 5
    assert o["comm_exposed_us"] == 20.0
    assert o["overlap_frac"] == round(45.0 / 65.0, 4)
    assert o["comm_gbs_active"] == round(65e3 / 65e-6 / 1e9, 1)   # 1 GB/s


def test_overlap_of_without_matmul_records_counts_everything_exposed():
    o = bench.overlap_of([(1, 0, 0.0, 3.0), (1, 1, 2.0, 5.0)], comm_bytes=1.0)
    assert o == {"comm_active_us": 5.0, "comm_hidden_us": 0.0, "comm_exposed_us": 5.0}


def test_mean_dicts_averages_the_numeric_keys_only():
    m = bench.mean_dicts([{"a": 1.0, "b": None, "c": 2}, {"a": 3.0, "b": 4.0, "c": 4}])
    assert m == {"a": 2.0, "c": 3.0}


def test_traffic_summary_matches_the_kernels_source():
    """The HBM traffic the bench line reports comes from the committed
    rocprofv3 summary, which names the kernels.hip it was taken on: after a
    kernel change the counters must be taken again (the bench reports null
    until then)."""
    t = bench.measured_traffic()
    assert t is not None, "profiles/ traffic summary was taken on another kernels.hip"
    fields = {}
    for line in open(bench.TRAFFIC_SUMMARY):
        if ":" in line and not line.startswith(("#", "|", " ", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    assert t == float(fields["traffic_bytes_per_launch"])
    assert t >= float(fields["algorithmic_bytes_per_launch"])


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""
