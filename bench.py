"""Benchmark of one mixed chunked-prefill step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is the append of the new tokens' K/V followed by the attention over one
synthetic batch already resident in HBM: one hybrid_step_fwd call (default), or
paged_kv_append then hybrid_attn_fwd (--entry calls).  Default workload: 2
prefill chunks of 512 (histories 0 and 1536) + 30 decodes with history
U[512, 4096], 32 heads x 128, bf16, 16-token pages, shuffled block ids.  Prints
ONE JSON line: microseconds per step, the fraction of the step roofline
max(FLOPs / MFMA peak, bytes / HBM peak), a roofline object for the timed call
(HIP events on the stream it runs on) and the CPU oracle's time on the host
cores as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "µs per mixed step + KV GB/s & TFLOP/s as % of step roofline (1 MI355X)"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def algorithmic_work(meta, spec):
    """FLOPs and bytes the method must move, independent of the implementation.

    FLOPs = 4 * D * Hq * (visible (query, key) pairs); bytes count every KV
    element once, Q in, O out, the append's read and write of the new K/V, and
    the int32 metadata."""
    lq = np.diff(meta.cu_seqlens_q).astype(np.int64)
    lk = meta.seqlens_k.astype(np.int64)
    vis = lq * (lk - lq) + lq * (lq + 1) // 2
    d, hq, hkv = spec.head_dim, spec.num_heads, spec.num_kv_heads
    e = 4 if spec.dtype == "f32" else 2
    t = int(lq.sum())
    b = len(lk)
    flops = 4.0 * d * hq * float(vis.sum())
    kv_bytes = e * d * hkv * 2.0 * float(lk.sum())
    qo_bytes = e * d * 2.0 * hq * t
    append_bytes = e * d * 4.0 * hkv * t
    meta_bytes = 4.0 * (float(((lk + 15) // 16).sum()) + 2 * b + 1 + t)
    attn_bytes = kv_bytes + qo_bytes + 4.0 * (float(((lk + 15) // 16).sum()) + 2 * b + 1)
    return {"flops": flops, "kv_bytes": kv_bytes, "attn_bytes": attn_bytes,
            "append_bytes": append_bytes + 4.0 * t,
            "step_bytes": kv_bytes + qo_bytes + append_bytes + meta_bytes}


def profiled_traffic(workload_name, unit):
    """HBM bytes per timed call (unit "step": hybrid_step_fwd; "attn": the
    attention call) from the committed rocprofv3 counter summary of this
    workload, or None when there is none or the kernel sources changed since
    the counters were taken."""
    import hashlib
    from pathlib import Path
    root = Path(__file__).resolve().parent
    name = f"step_{workload_name}" if unit == "step" else f"attn_kernel_{workload_name}"
    prof = root / "profiles" / f"{name}.txt"
    if not prof.exists():
        return None
    fields = dict(line.split(": ", 1) for line in prof.read_text().splitlines()
                  if line.startswith(("source_sha256: ", "traffic_bytes: ")))
    h = hashlib.sha256()
    for src in ("attention.hip", "ha_common.hpp", "ha_internal.hpp"):
        h.update((root / "chunked_prefill_mixed_hybrid_amd" / "csrc" / src).read_bytes())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return float(fields["traffic_bytes"])


def cpu_baseline(ds, spec, meta, budget_s=10.0):
    """The oracle (as it stands) on the host cores: the whole step (append +
    attention for every row), repeated until about budget_s of CPU time."""
    import oracle
    from chunked_prefill_mixed_hybrid_amd import workload as W
    orc = oracle.default()
    kc0, vc0 = W.to_host_array(ds.k_cache), W.to_host_array(ds.v_cache)
    q, key, value = (W.to_host_array(x) for x in (ds.q, ds.key, ds.value))
    runs, t_total = 0, 0.0
    while t_total < budget_s and runs < 100:
        kc, vc = kc0.copy(), vc0.copy()
        t0 = time.perf_counter()
        orc.append(key, value, meta.slot_mapping, kc, vc)
        orc.attention(q, kc, vc, meta.cu_seqlens_q, meta.seqlens_k, meta.block_table)
        t_total += time.perf_counter() - t0
        runs += 1
    return {"value": round(1e6 * t_total / runs, 1), "unit": "us/step",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"the whole step (append + every row), {runs} run(s), fp64 oracle"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps each preceded by a 1 GiB cache-flush write")
    ap.add_argument("--launch", default="fused", choices=["fused", "serial", "two-streams"],
                    help="fused: hybrid_attn_fwd; serial / two-streams: the two-launch baseline")
    ap.add_argument("--entry", default="step", choices=["step", "calls"],
                    help="step: one hybrid_step_fwd call per step; calls: paged_kv_append, then "
                         "the attention call")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from chunked_prefill_mixed_hybrid_amd import binding as B
    from chunked_prefill_mixed_hybrid_amd import workload as W

    B.load()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    spec, meta = W.make_step(args.config, args.seed)
    ds = W.device_values(spec, meta, seed=args.seed)
    out = torch.empty_like(ds.q)
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, spec.num_heads,
                           spec.head_dim)
    stream = torch.cuda.Stream()
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def attention():
        if args.launch == "fused":
            B.hybrid_attn_fwd(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q, ds.seqlens_k,
                              ds.block_table, meta.max_seqlen_q, meta.max_seqlen_k, out=out,
                              workspace=ws, stream=stream)
        else:
            B.hybrid_attn_fwd_two_launch(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q,
                                         ds.seqlens_k, ds.block_table, meta.max_seqlen_q,
                                         meta.max_seqlen_k, out=out, workspace=ws,
                                         two_streams=args.launch == "two-streams", stream=stream)

    one_call = args.entry == "step" and args.launch == "fused"

    def step():
        if one_call:
            B.hybrid_step_fwd(ds.key, ds.value, ds.slot_mapping, ds.q, ds.k_cache, ds.v_cache,
                              ds.cu_seqlens_q, ds.seqlens_k, ds.block_table, meta.max_seqlen_q,
                              meta.max_seqlen_k, out=out, workspace=ws, stream=stream)
            return
        B.paged_kv_append(ds.key, ds.value, ds.slot_mapping, ds.k_cache, ds.v_cache, stream=stream)
        attention()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # timed region: exactly K steps back to back on one stream, nothing else enqueued
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = t_start.elapsed_time(t_end)

    # the timed call on its own (HIP events on the stream the kernels run on)
    call_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for e0, e1 in call_ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([e0.elapsed_time(e1) for e0, e1 in call_ev])

    # the append and the attention call separately (reference), a further pass
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1, e2 in ev:
        e0.record(stream)
        B.paged_kv_append(ds.key, ds.value, ds.slot_mapping, ds.k_cache, ds.v_cache, stream=stream)
        e1.record(stream)
        attention()
        e2.record(stream)
    torch.cuda.synchronize()
    attn_ms = np.array([e1.elapsed_time(e2) for _, e1, e2 in ev])
    append_ms = np.array([e0.elapsed_time(e1) for e0, e1, _ in ev])
    step_ms = np.array([e0.elapsed_time(e2) for e0, _, e2 in ev])

    # cold steps: a 1 GiB write before each step evicts L2 and the 256 MB MALL
    cold = []
    for _ in range(args.cold_steps):
        with torch.cuda.stream(stream):
            flush_buf.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))

    if args.calibrate_copy:  # a copy of known size: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = algorithmic_work(meta, spec)
    us_step = 1e6 * wall / args.steps
    peak_tf = PEAK_MFMA_TFLOPS[spec.dtype]
    t_mfma_us = w["flops"] / (peak_tf * 1e12) * 1e6
    t_hbm_us = w["step_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e6
    roof_us = max(t_mfma_us, t_hbm_us)
    attn_us = float(np.mean(attn_ms)) * 1e3
    # the roofline unit: the whole step call (append + attention) with the step's
    # bytes, or the attention call with its own bytes when the two are separate
    unit_us = float(np.mean(call_ms)) * 1e3 if one_call else attn_us
    unit_bytes = w["step_bytes"] if one_call else w["attn_bytes"]
    attn_bound = "hbm" if unit_bytes / (PEAK_HBM_GBS * 1e9) >= w["flops"] / (peak_tf * 1e12) else "mfma"
    if attn_bound == "hbm":
        achieved = unit_bytes / (unit_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        achieved = w["flops"] / (unit_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4), "traffic": None}
    if one_call:
        roof["kernel"] = ("hybrid_step_fwd (append + planner in one launch, attn_kernel, combine_kernel, "
                          "back to back)")
    elif args.launch == "fused":
        roof["kernel"] = "hybrid_attn_fwd (plan_kernel + attn_kernel + combine_kernel, back to back)"
    else:
        roof["kernel"] = (f"hybrid_attn_fwd_two_launch ({args.launch}: plan, chunk launch, decode launch, "
                          "combine)")
    roof["avg_us"] = round(unit_us, 2)
    roof["traffic"] = profiled_traffic(spec.name, "step" if one_call else "attn") \
        if args.launch == "fused" else None

    result = {
        "metric": METRIC, "value": round(us_step, 2), "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us_step / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": spec.name, "num_seqs": meta.num_seqs, "total_q": meta.total_q,
                   "num_heads": spec.num_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "page_size": meta.page_size,
                   "max_seqlen_q": meta.max_seqlen_q, "max_seqlen_k": meta.max_seqlen_k,
                   "seed": args.seed, "launch": args.launch,
                   "entry": "hybrid_step_fwd" if one_call else "paged_kv_append + attention"},
        "gpu_us_per_step": round(1e3 * gpu_ms / args.steps, 2),
        "tflops": round(w["flops"] / (us_step * 1e-6) / 1e12, 2),
        "kv_gbps": round(w["kv_bytes"] / (us_step * 1e-6) / 1e9, 1),
        "step_gbps": round(w["step_bytes"] / (us_step * 1e-6) / 1e9, 1),
        "step_roofline_us": round(roof_us, 2),
        "frac_step_roofline": round(roof_us / us_step, 4),
        "append_us": round(float(np.mean(append_ms)) * 1e3, 2),
        "attn_us": round(attn_us, 2),
        "cold_us_per_step": round(float(np.median(cold)) * 1e3, 2) if cold else None,
        "step_us_percentiles": percentiles(call_ms if one_call else step_ms),
        "cold_us_percentiles": percentiles(np.array(cold)) if cold else None,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ds, spec, meta)
    print(json.dumps(result), flush=True)


def percentiles(ms):
    """p10 / p50 / p90 of per-step durations given in ms, in us."""
    return {f"p{q}": round(float(np.percentile(ms, q)) * 1e3, 2) for q in (10, 50, 90)}


if __name__ == "__main__":
    main()
