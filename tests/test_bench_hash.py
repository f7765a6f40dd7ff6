"""The key that ties a profile record to the code it was measured on (bench.kernel_source_hash).

A counter record is reported as a kernel's traffic only while the hash of the sources that
decide that kernel matches. The hash must cover every kernel and host source and the build
flags, ignore comments and whitespace, and change with any code edit.
"""
from __future__ import annotations

import os
import shutil

import bench
from qk_rmsnorm_rope_amd import workloads as wl

CSRC = os.path.join(bench.ROOT, "qk_rmsnorm_rope_amd", "csrc")


def test_every_source_is_hashed():
    hashed = set(bench.COMMON_SOURCES + bench.PROLOGUE_SOURCES + bench.CAM_SOURCES)
    for f in os.listdir(CSRC):
        assert "qk_rmsnorm_rope_amd/csrc/" + f in hashed, f
    assert "qk_rmsnorm_rope_amd/build.py" in hashed


def test_every_record_matches_the_current_sources():
    for w in wl.WORKLOADS.values():
        assert bench.traffic_from_profile(w) is not None, w.name


def test_comments_do_not_change_the_hash_and_code_does(tmp_path, monkeypatch):
    for rel in set(bench.COMMON_SOURCES + bench.PROLOGUE_SOURCES + bench.CAM_SOURCES):
        os.makedirs(tmp_path / os.path.dirname(rel), exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, rel), tmp_path / rel)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    w3, cam = wl.WORKLOADS["rope3d_neox_fp8_b2_s18480_h20_d64"], wl.WORKLOADS["cam_prep_b2_s18480_h20_d64"]
    h3, hc = bench.kernel_source_hash(w3), bench.kernel_source_hash(cam)
    wrap = tmp_path / "qk_rmsnorm_rope_amd/csrc/qkrope_kernels_3d_d64.hip"
    build = tmp_path / "qk_rmsnorm_rope_amd/build.py"
    wrap.write_text(wrap.read_text() + "\n// a comment\n/* and\n another */\n\n")
    build.write_text(build.read_text() + "\n# a comment\n")
    assert bench.kernel_source_hash(w3) == h3 and bench.kernel_source_hash(cam) == hc
    wrap.write_text(wrap.read_text().replace("namespace qkrope", "namespace  qkrope", 1))
    assert bench.kernel_source_hash(w3) == h3           # whitespace only
    wrap.write_text(wrap.read_text() + "static int planted;\n")
    assert bench.kernel_source_hash(w3) != h3           # code in a prologue wrapper
    assert bench.kernel_source_hash(cam) == hc          # does not touch the camera's key
    build.write_text(build.read_text().replace("-O3", "-O2"))
    assert bench.kernel_source_hash(cam) != hc          # build flags key every kernel
