"""ctypes front end of the C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Arrays are host
numpy arrays; bf16 data is passed as its raw uint16 bit pattern.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
LIB_NAME = "liboracle.so"
F32, BF16 = 0, 1

_i32p = ctypes.POINTER(ctypes.c_int32)


def build(src: Path | None = None, out: Path | None = None, quiet: bool = True) -> Path:
    """Compile the oracle with gcc (plain -O2, no fp contraction, OpenMP)."""
    src = Path(src) if src else HERE / "oracle.c"
    out = Path(out) if out else HERE / LIB_NAME
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-std=c99", "-Wall", "-I", str(HERE), str(src), "-o", str(out) + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    os.replace(str(out) + ".tmp", out)
    return out


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle stores float32 or bf16-as-uint16, got {a.dtype}")


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class Oracle:
    """One loaded copy of the oracle library (the real one, or a test mutant)."""

    def __init__(self, path: Path | str | None = None):
        # ORACLE_LIB names another build of oracle.c to load by default (the
        # sanitizer test runs the pins against an ASan/UBSan build this way)
        path = Path(path or os.environ.get("ORACLE_LIB") or HERE / LIB_NAME)
        if not path.exists():
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(str(path))
        lib.oracle_visible_counts.argtypes = [_i32p, _i32p, ctypes.c_int32, _i32p]
        lib.oracle_check_slots.argtypes = [_i32p, _i32p, _i32p, _i32p] + [ctypes.c_int32] * 4
        lib.oracle_append.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int32] * 6
        lib.oracle_attention.argtypes = ([ctypes.c_void_p] * 3 + [_i32p] * 3 + [ctypes.c_int32] * 7
                                         + [ctypes.c_double, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p])
        lib.oracle_num_threads.argtypes = []
        for f in ("oracle_visible_counts", "oracle_check_slots", "oracle_append",
                  "oracle_attention", "oracle_num_threads"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib

    # -- metadata -----------------------------------------------------------------
    def visible_counts(self, cu_seqlens_q, seqlens_k) -> np.ndarray:
        cu, sk = _i32(cu_seqlens_q), _i32(seqlens_k)
        out = np.zeros(int(cu[-1]), dtype=np.int32)
        rc = self.lib.oracle_visible_counts(cu.ctypes.data_as(_i32p), sk.ctypes.data_as(_i32p),
                                            len(sk), out.ctypes.data_as(_i32p))
        if rc != 0:
            raise ValueError(f"oracle_visible_counts: invalid segments (rc={rc})")
        return out

    def check_slots(self, cu_seqlens_q, seqlens_k, block_table, slot_mapping, page_size,
                    num_blocks) -> int:
        cu, sk, bt, sm = (_i32(cu_seqlens_q), _i32(seqlens_k), _i32(block_table),
                          _i32(slot_mapping))
        return self.lib.oracle_check_slots(cu.ctypes.data_as(_i32p), sk.ctypes.data_as(_i32p),
                                           bt.ctypes.data_as(_i32p), sm.ctypes.data_as(_i32p),
                                           len(sk), bt.shape[1], page_size, num_blocks)

    # -- append -------------------------------------------------------------------
    def append(self, key, value, slot_mapping, k_cache, v_cache) -> None:
        """In place: writes key/value [T, Hkv, D] into caches [NB, P, Hkv, D]."""
        dt = _dtype_code(k_cache)
        assert key.dtype == value.dtype == v_cache.dtype == k_cache.dtype
        nb, p, hkv, d = k_cache.shape
        sm = _i32(slot_mapping)
        rc = self.lib.oracle_append(_ptr(key), _ptr(value), _ptr(sm), _ptr(k_cache),
                                    _ptr(v_cache), len(sm), hkv, d, p, nb, dt)
        if rc != 0:
            raise ValueError(f"oracle_append: slot out of range (rc={rc})")

    # -- attention ----------------------------------------------------------------
    def attention(self, q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                  scale: float | None = None, row_select=None, out=None) -> np.ndarray:
        """fp64 [T, Hq, D] output of the right-aligned causal paged attention."""
        dt = _dtype_code(q)
        assert k_cache.dtype == v_cache.dtype == q.dtype
        t, hq, d = q.shape
        nb, p, hkv, d2 = k_cache.shape
        assert d == d2
        cu, sk, bt = _i32(cu_seqlens_q), _i32(seqlens_k), _i32(block_table)
        assert cu[-1] == t
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        if out is None:
            out = np.full((t, hq, d), np.nan, dtype=np.float64)
        sel = None
        if row_select is not None:
            sel = np.ascontiguousarray(row_select, dtype=np.uint8)
            assert sel.shape == (t,)
        rc = self.lib.oracle_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       cu.ctypes.data_as(_i32p), sk.ctypes.data_as(_i32p),
                                       bt.ctypes.data_as(_i32p), len(sk), hq, hkv, d, p, nb,
                                       bt.shape[1], float(scale), dt, _ptr(sel), _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle_attention: invalid input (rc={rc})")
        return out

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
