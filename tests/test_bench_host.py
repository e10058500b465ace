"""Host checks of bench.py: the algorithmic work behind the roofline figures,
and the refusal of more than one GPU."""
import subprocess
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent.parent


def _visible_pairs(meta):
    # count (query, key) pairs one row at a time from the mask definition: row i
    # of a segment with Lq rows and Lk keys sees keys 0 .. Lk - Lq + i
    cu, lk = meta.cu_seqlens_q, meta.seqlens_k
    total = 0
    for b in range(len(lk)):
        lq = int(cu[b + 1] - cu[b])
        total += int(np.sum(np.arange(lq, dtype=np.int64) + (int(lk[b]) - lq) + 1))
    return total


def test_worked_example_work():
    import bench
    from chunked_prefill_mixed_hybrid_amd import workload as W
    spec, meta = W.make_step(1, 0)
    work = bench.algorithmic_work(meta, spec)
    pairs = _visible_pairs(meta)
    assert pairs == 121 + 46 + sum(8192 + i + 1 for i in range(1808))
    assert work["flops"] == 4.0 * 64 * 2 * pairs           # QK^T and P.V, 2 heads x 64
    assert abs(work["flops"] - 8.42e9) < 0.01e9
    # every K/V element once, Q in and O out, the append's read and write, int32 metadata
    keys = 121 + 46 + 10000
    pages = -(-121 // 16) + -(-46 // 16) + -(-10000 // 16)
    expect = 4 * 64 * (2 * 2 * keys + 2 * 2 * 1810 + 4 * 2 * 1810) + 4 * (pages + 2 * 3 + 1 + 1810)
    assert work["step_bytes"] == expect
    assert abs(work["step_bytes"] - 16.0e6) < 0.1e6
    # step roofline: MFMA-bound at the fp32 peak
    assert abs(work["flops"] / (bench.PEAK_MFMA_TFLOPS["f32"] * 1e12) * 1e6 - 53.5) < 0.1


def test_mixed_step_work_is_hbm_bound():
    import bench
    from chunked_prefill_mixed_hybrid_amd import workload as W
    spec, meta = W.make_step(2, 0)
    work = bench.algorithmic_work(meta, spec)
    assert work["flops"] == 4.0 * 128 * 32 * _visible_pairs(meta)
    t_hbm = work["step_bytes"] / (bench.PEAK_HBM_GBS * 1e9)
    t_mfma = work["flops"] / (bench.PEAK_MFMA_TFLOPS["bf16"] * 1e12)
    assert t_hbm > 10 * t_mfma
    assert abs(t_hbm * 1e6 - 159.5) < 1.0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
