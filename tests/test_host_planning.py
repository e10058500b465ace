"""Planning arithmetic shared by the launcher and the kernels, checked on the
host: tests/host_planning_check.cpp includes csrc/ha_internal.hpp, is built
with hipcc (host code only) and run here."""
import os
import subprocess
from pathlib import Path

import pytest

from chunked_prefill_mixed_hybrid_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.hipcc()), reason="hipcc not available")


def test_host_planning(tmp_path: Path):
    src = Path(__file__).with_name("host_planning_check.cpp")
    exe = tmp_path / "host_planning_check"
    res = subprocess.run([build.hipcc(), f"--offload-arch={build.ARCH}", "-std=c++17", "-O2",
                          f"-I{build.CSRC}", f"-I{build.INCLUDE}",
                          str(src), "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "passed" in run.stdout
