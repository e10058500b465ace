"""The oracle and the host step generator under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

oracle.c and the host-only sources of the library (csrc/scheduler.cpp,
csrc/status.cpp) are rebuilt with -fsanitize=address,undefined, and the oracle
pins and the scheduler tests (random traces included, and the oracle run over
scheduled steps) run against those builds in a child process with the
sanitizer runtimes preloaded; any report ends that process with an error.
The planted-mistake mutants are not run here: some of them index outside the
pool on purpose, which is what their pins catch."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

from chunked_prefill_mixed_hybrid_amd import build

ROOT = Path(__file__).resolve().parent.parent
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                    reason="gcc sanitizer runtimes not installed")
def test_oracle_and_scheduler_under_sanitizers(tmp_path):
    oracle_lib = tmp_path / "liboracle_san.so"
    host_lib = tmp_path / "libhost_san.so"
    cmds = [
        ["gcc", *SAN, "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
         "-I", str(ROOT / "oracle"), str(ROOT / "oracle" / "oracle.c"), "-o", str(oracle_lib), "-lm"],
        ["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", f"-I{build.INCLUDE}",
         str(build.CSRC / "scheduler.cpp"), str(build.CSRC / "status.cpp"), "-o", str(host_lib)],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
    report = tmp_path / "used.txt"
    env = dict(os.environ,
               LD_PRELOAD=f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               ORACLE_LIB=str(oracle_lib), HA_SAN_HOST_LIB=str(host_lib), HA_SAN_REPORT=str(report),
               PYTHONPATH=os.pathsep.join([str(ROOT / "tests"), str(ROOT)]))
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "-p", "sanitize_plugin", "-m", "not gpu",
                          str(ROOT / "tests" / "test_oracle_pins.py"),
                          str(ROOT / "tests" / "test_scheduler.py")],
                         cwd=str(ROOT), env=env, capture_output=True, text=True, timeout=900)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    used = report.read_text()
    assert f"oracle {oracle_lib}" in used and f"host {host_lib}" in used, used


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc sanitizer runtimes not installed")
def test_sanitizer_reports_a_planted_overrun(tmp_path):
    """The same build and preload on a copy of oracle.c whose first pass reads
    one score past the visible keys: the child process must report it."""
    src = (ROOT / "oracle" / "oracle.c").read_text()
    anchor = "if (s[j] > m) m = s[j];\n      }"
    assert src.count(anchor) == 1
    bad = tmp_path / "oracle_overrun.c"
    bad.write_text(src.replace(anchor, anchor + "\n      m = fmax(m, s[max_lk]);"))
    lib = tmp_path / "liboracle_overrun.so"
    r = subprocess.run(["gcc", *SAN, "-fopenmp", "-fPIC", "-shared", "-std=c99", "-I", str(ROOT / "oracle"),
                        str(bad), "-o", str(lib), "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    code = ("import numpy as np, oracle\n"
            "o = oracle.Oracle()\n"
            "q = np.ones((1, 1, 8), np.float32); kc = np.ones((1, 16, 1, 8), np.float32)\n"
            "o.attention(q, kc, kc.copy(), [0, 1], [3], np.zeros((1, 1), np.int32))\n")
    env = dict(os.environ, LD_PRELOAD=_runtime("libasan.so"), ASAN_OPTIONS="detect_leaks=0",
               ORACLE_LIB=str(lib), PYTHONPATH=str(ROOT))
    run = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=300)
    assert run.returncode != 0 and "heap-buffer-overflow" in run.stderr, run.stderr[-2000:]
