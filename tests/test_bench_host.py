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


def test_long_context_step_is_hbm_bound():
    """The headline workload: 1024-token chunk at history 130048 + 64 decodes
    (seed-0 histories), 32 x 128 bf16."""
    import bench
    from chunked_prefill_mixed_hybrid_amd import workload as W
    spec, meta = W.make_step(4, 0)
    work = bench.algorithmic_work(meta, spec)
    pairs = _visible_pairs(meta)
    assert work["flops"] == 4.0 * 128 * 32 * pairs
    chunk_pairs = sum(130048 + i + 1 for i in range(1024))
    assert pairs == chunk_pairs + int(meta.seqlens_k[1:].sum())
    roof, bound = bench.step_roofline_us(work, spec)
    assert bound == "hbm" and abs(roof - work["step_bytes"] / 8e12 * 1e6) < 1e-6
    assert 9400 < roof < 9700


def test_full_prefill_is_mfma_bound():
    """The 10000-token prompt in one step, 64 x 128 bf16: causal pairs
    10000 * 10001 / 2, MFMA-bound at 2.5 PFLOP/s."""
    import bench
    from chunked_prefill_mixed_hybrid_amd import workload as W
    spec, meta = W.make_step("5b", 0)
    work = bench.algorithmic_work(meta, spec)
    assert work["flops"] == 4.0 * 128 * 64 * (10000 * 10001 // 2)
    roof, bound = bench.step_roofline_us(work, spec)
    assert bound == "mfma" and abs(roof - 655.4) < 0.1


def test_cpu_baseline_sample_scales_by_pairs():
    """The oracle baseline on a small step held in CPU tensors: whole-step mode,
    then sample mode (forced by a tiny host-memory bound) -- both report the
    core count, the CPU model and what was timed."""
    import bench
    from chunked_prefill_mixed_hybrid_amd import workload as W
    segs = [(1, 900), (200, 1400), (1, 40), (1, 2000)]
    spec, meta = W.custom_step(segs, 2, 2, 64, W.F32, seed=3)
    ds = W.device_values(spec, meta, seed=3, device="cpu")
    w = bench.algorithmic_work(meta, spec)
    full = bench.cpu_baseline(ds, spec, meta, w, budget_s=0.0)
    assert "whole step" in full["sample"] and full["value"] > 0
    part = bench.cpu_baseline(ds, spec, meta, w, budget_s=0.0, max_host_bytes=800 * 1024,
                              target_pairs_heads=2e4)
    assert "chunk rows" in part["sample"] and part["value"] > 0
    for r in (full, part):
        assert r["kind"] == "oracle" and r["cores"] >= 1 and r["host_cores"] >= 1
        assert isinstance(r["cpu_model"], str)
