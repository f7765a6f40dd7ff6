"""bench.py's result line, as far as it can be checked without a GPU: the refusal of more than one
GPU, the headline workload and its sub-records, and the roofline object (fields, arithmetic, and
the counter traffic taken from the committed record of the current sources)."""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
bench = pytest.importorskip("bench")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_headline_is_the_largest_single_gpu_3d_workload_with_configs_3_and_4_and_the_camera_beside_it():
    named_3d = [w for w in wl.WORKLOADS.values()
                if bench.is_3d(w) and not bench.is_sharded(w) and not bench.is_cam(w)]
    largest = max(named_3d, key=bench.algorithmic_bytes)
    assert bench.DEFAULT_WORKLOAD == largest.name == "rope3d_yarn_nonorm_s122880_h16_d256"
    assert set(bench.ALSO_TIMED) == {"rope3d_across_interleaved_s15360_h32_d128",
                                     "rope3d_neox_fp8_b2_s18480_h20_d64",
                                     "cam_prep_b2_s18480_h20_d64"}


@pytest.mark.parametrize("name", [bench.DEFAULT_WORKLOAD, *bench.ALSO_TIMED])
def test_roofline_fields_and_arithmetic(name):
    w = wl.WORKLOADS[name]
    mean_launch = 1e-3
    r = bench.roofline(w, mean_launch)
    assert {"bound", "achieved", "peak", "unit", "frac", "traffic"} <= set(r)
    assert (r["bound"], r["peak"], r["unit"]) == ("hbm", 8000.0, "GB/s")
    assert r["achieved"] == pytest.approx(bench.algorithmic_bytes(w) / mean_launch / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    # traffic: the calibrated FETCH_SIZE + WRITE_SIZE bytes of the committed record
    text = open(os.path.join(ROOT, "profiles", f"counters_{name}.md"), encoding="utf-8").read()
    rec = json.loads(re.search(r"<!-- traffic (\{.*\}) -->", text).group(1))
    assert r["traffic"] == rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    # the camera prologue's head groups re-read their tokens' matrices and table rows: 2% more
    # reads than its algorithmic bytes (one pass) on the contiguous layout
    assert abs(r["traffic"] / r["algorithmic_bytes"] - 1) < (0.03 if bench.is_cam(w) else 0.01)
