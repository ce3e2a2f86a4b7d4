"""The read-ahead template, compiled for the host and checked on every depth,
drain form and loop length (tests/pipeline_check.cpp states the contract)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "int8_dequant_dot_amd", "csrc")


@pytest.mark.parametrize("opt", ["-O0", "-O2"])
def test_read_ahead_contract(tmp_path, opt):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "pipeline_check"
    subprocess.run([cxx, "-std=c++17", opt, "-Wall", "-Wno-unknown-pragmas", "-I", CSRC,
                    os.path.join(HERE, "pipeline_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) == 2 * sum(4 * d + 6 for d in (1, 2, 3, 4, 5, 6, 7, 8, 16, 32))
