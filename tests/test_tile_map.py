"""CPU check of the grouped GEMMs' tile assignment: builds tile_map_check.hip
(which includes the GEMM source and calls its host-callable assign_tile) with
hipcc and runs it. Over thousands of random expert-count patterns, shapes,
split limits and CU counts it checks that the launched grid hands every tile
to exactly one workgroup, whole or as both halves. Needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_assignment_covers_every_tile(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "tests", "tile_map_check.hip")
    exe = str(tmp_path / "tile_map_check")
    build = subprocess.run(
        [hipcc, "-O2", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "sparse_mixture_experts_renorm_amd", "csrc"),
         "-I", os.path.join(ROOT, "include"), src, "-o", exe],
        capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0 and run.stdout.startswith("ok"), run.stdout + run.stderr
