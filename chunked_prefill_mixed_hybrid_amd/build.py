"""Build libhybridattn.so (hand-written HIP for gfx950) in the package directory.

    python -m chunked_prefill_mixed_hybrid_amd.build

Each .hip translation unit is compiled with hipcc for gfx950 only, the host-only
C++ (the step generator) with g++, then everything is linked into one shared
library exporting the C ABI of include/hybrid_attn.h and include/ha_scheduler.h.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libhybridattn.so"
SOURCES = ["api.hip", "attention.hip", "kv_append.hip"]
HOST_SOURCES = ["scheduler.cpp", "status.cpp"]  # host-only C++ (no device code), built with the host compiler
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # never emit packed fp32 VALU ops (v_pk_*_f32): plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the one-segment prefill kernel rescales its
    # output accumulators with VALU multiplies, and with AGPR accumulators the
    # compiler copied all 128 of them out and back on every key block, taken
    # branch or not (the other kernels compile to the same code either way)
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return str(Path(rocm) / "bin" / "hipcc")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = [l for l in (res.stdout + res.stderr).splitlines()
             if "packed-fp32-ops" not in l]  # host pass does not know the GPU feature
    if res.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> Path:
    obj_dir = PKG / "_build"
    obj_dir.mkdir(exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = obj_dir / (Path(src).stem + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", str(CSRC / src),
                     "-o", str(obj)])
    for src in HOST_SOURCES:
        obj = obj_dir / (Path(src).stem + ".o")
        objs.append(obj)
        cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}",
                     "-c", str(CSRC / src), "-o", str(obj)])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out:
                print(out)
    tmp = LIB.with_suffix(".so.tmp")
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
