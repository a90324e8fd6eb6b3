"""bench.py's host-side helpers (no GPU): the roofline record, the profile lookup of counted
HBM traffic (with its source-hash staleness check) and the CPU-baseline records."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_roofline_record():
    r = bench.roofline("hbm", 2000.0, 8000.0, "GB/s", 1234)
    assert r == {"bound": "hbm", "achieved": 2000.0, "peak": 8000.0, "unit": "GB/s", "frac": 0.25, "traffic": 1234}


@pytest.mark.parametrize("key", ["C1", "C2", "C3a_auto", "C3b_auto", "C4", "C4_split", "C5", "C5_fused", "MLA",
                                 "CASC_logsumexp", "CASC_topk_softmax", "CASCG_softmax", "CASCG_absmax"])
def test_every_bench_line_has_current_counted_traffic(key):
    """Each workload's profile summary exists, names the kernel sources it measured, and
    their hash matches the sources in the tree (else the bench would report traffic null)."""
    t = bench.profiled_traffic(key)
    assert isinstance(t, int) and t > 0


def test_unknown_workload_has_no_traffic():
    assert bench.profiled_traffic("no_such_workload") is None


def test_cpu_baseline_records():
    base, info = bench.cpu_baselines(["C1", "C4"], 0.05, 0.05)
    assert set(base) == {"C1", "C4"}
    for rec in base.values():
        assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["cores"] >= 1 and rec["sample"]
    assert base["C1"]["unit"] == "TFLOP/s" and base["C4"]["unit"] == "GB/s"
    assert info["usable_cpus"] >= 1 and "cpu_model" in info
