"""The chunk-walking matmul's workgroup schedule (csrc/coc_schedule.h), built
for the host with g++ and checked against brute-force definitions: every tile
once, per-workgroup order, the two-round split, the gatherer numbering, the
chunks the first round waits for."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "tensor_gemm_collective_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_schedule_against_definitions(tmp_path):
    exe = str(tmp_path / "schedule_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC, os.path.join(HERE, "schedule_check.cpp"),
                    "-o", exe], check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("bad 0"), out.stdout
