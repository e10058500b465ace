"""Benchmark of one mixed chunked-prefill step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--extra 1,2,3,5a,5b]

A step is the append of the new tokens' K/V followed by the attention over one
synthetic batch already resident in HBM: one hybrid_step_fwd call (default), or
paged_kv_append then hybrid_attn_fwd (--entry calls).  The headline workload
is the largest single-GPU step: a chunk of 1024 tokens at history 130048 of a
131072-token prompt plus 64 decodes with history U[8192, 131072], 32 heads x
128, bf16, 16-token pages, shuffled block ids (75 GB of pages).

Timed region: K steps on one stream, each preceded by a 1 GiB read that
evicts L2 and the 256 MB MALL (cold, as a serving step meets its KV), each
bracketed by HIP events; `value` is the median step in microseconds.  Also
reported: the same steps back to back (warm), the same steps after a 1 GiB
write instead (whose dirty lines are written back during the step), the fraction of the step roofline
max(FLOPs / MFMA peak, bytes / HBM peak), a roofline object for the attention
call (HIP events on the stream its kernels run on), the CPU oracle's time on
the host cores as a baseline (a bounded sample of the step, scaled by the
number of (query, key) pairs), and the other workloads' cold and warm times.
Prints ONE JSON line.
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
FLUSH_BYTES = 1 << 30


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
            "step_bytes": kv_bytes + qo_bytes + append_bytes + meta_bytes,
            "pairs": vis}


def step_roofline_us(w, spec):
    t_mfma = w["flops"] / (PEAK_MFMA_TFLOPS[spec.dtype] * 1e12) * 1e6
    t_hbm = w["step_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e6
    return max(t_mfma, t_hbm), ("mfma" if t_mfma > t_hbm else "hbm")


def profiled_traffic(workload_name):
    """HBM bytes per attention call from the committed rocprofv3 counter
    summary of this workload, or None when there is none or the kernel sources
    changed since the counters were taken."""
    import hashlib
    from pathlib import Path
    root = Path(__file__).resolve().parent
    prof = root / "profiles" / f"attn_kernel_{workload_name}.txt"
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(ds, spec, meta, w, budget_s=15.0, max_host_bytes=6 << 30, target_pairs_heads=1e9):
    """The oracle (as it stands) on the host cores.  Steps whose pages fit
    max_host_bytes and whose work is small run whole (append + every row);
    bigger ones run a bounded sample -- evenly spaced rows of the chunk
    segments plus a seeded subset of the decode segments, pages within
    max_host_bytes -- and the time is scaled to the whole step by the ratio of
    (query, key) pairs x heads, the oracle's unit of work.  Repeated until
    about budget_s of wall time (at least once); the page copy to the host is
    not timed."""
    import oracle
    from oracle import sample as OS
    orc = oracle.default()
    lq = np.diff(meta.cu_seqlens_q).astype(np.int64)
    lk = meta.seqlens_k.astype(np.int64)
    pairs = w["pairs"]
    e = 4 if spec.dtype == "f32" else 2
    key_bytes = spec.num_kv_heads * spec.head_dim * e
    seg_bytes = 2 * ((lk + 15) // 16) * 16 * key_bytes
    total_ph = float(pairs.sum()) * spec.num_heads
    whole = float(seg_bytes.sum()) <= max_host_bytes and total_ph <= 4 * target_pairs_heads
    sel = np.zeros(meta.total_q, np.uint8)
    if whole:
        segs = list(range(meta.num_seqs))
        sel[:] = 1
        what = "the whole step (append + every row)"
    else:
        rng = np.random.default_rng(7)
        chunks = [b for b in range(meta.num_seqs) if lq[b] > 1]
        decs = [b for b in range(meta.num_seqs) if lq[b] == 1]
        segs, used, ph = [], 0, 0.0
        n_rows = 0
        for b in chunks:  # evenly spaced rows of every chunk, up to 70 % of the target
            if used + seg_bytes[b] > max_host_bytes:
                continue
            r0, n = int(meta.cu_seqlens_q[b]), int(lq[b])
            h0 = int(lk[b] - n)
            per_row = (h0 + np.arange(n) + 1) * float(spec.num_heads)
            take = max(1, min(n, int(0.7 * target_pairs_heads / max(1.0, per_row.mean()))))
            rows = np.unique(np.linspace(0, n - 1, take).round().astype(np.int64))
            sel[r0 + rows] = 1
            ph += float(per_row[rows].sum())
            n_rows += len(rows)
            segs.append(b)
            used += int(seg_bytes[b])
        n_dec = 0
        for b in rng.permutation(decs):  # then decodes, while pages and work allow
            if used + seg_bytes[b] > max_host_bytes or ph >= target_pairs_heads:
                continue
            sel[int(meta.cu_seqlens_q[b])] = 1
            ph += float(lk[b]) * spec.num_heads
            segs.append(int(b))
            used += int(seg_bytes[b])
            n_dec += 1
        segs.sort()
        what = (f"{n_rows} of {int(lq[chunks].sum())} chunk rows (evenly spaced) and {n_dec} of "
                f"{len(decs)} decode segments (seeded pick), with the append of their tokens; "
                f"{100.0 * ph / total_ph:.2f} % of the step's (query, key) pairs x heads, "
                f"time scaled by that ratio")
    smp = OS.SampledStep(meta, ds.q, ds.key, ds.value, ds.k_cache, ds.v_cache, segs)
    rs = sel[smp.rows]
    sample_ph = 0.0  # (query, key) pairs x heads of the selected rows
    for b in segs:
        r0, n = int(meta.cu_seqlens_q[b]), int(lq[b])
        rows = np.flatnonzero(sel[r0:r0 + n])
        sample_ph += float((lk[b] - n + rows + 1).sum()) * spec.num_heads
    runs, t_total = 0, 0.0
    while runs == 0 or (t_total < budget_s and runs < 100):
        kc, vc = smp.kc.copy(), smp.vc.copy()
        t0 = time.perf_counter()
        orc.append(smp.key, smp.value, smp.slot_mapping, kc, vc)
        orc.attention(smp.q, kc, vc, smp.cu, smp.sk, smp.block_table, row_select=None if whole else rs)
        t_total += time.perf_counter() - t0
        runs += 1
    per_run = t_total / runs
    return {"value": round(1e6 * per_run * total_ph / sample_ph, 1), "unit": "us/step",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{what}; fp64 oracle, {runs} run(s) of {per_run:.2f} s",
            "host_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "measured_s": round(t_total, 2)}


class Runner:
    """One workload resident on the device, and the calls that time it."""

    def __init__(self, config, seed, launch, entry, stream):
        import torch
        from chunked_prefill_mixed_hybrid_amd import binding as B
        from chunked_prefill_mixed_hybrid_amd import workload as W
        self.B, self.torch = B, torch
        self.spec, self.meta = W.make_step(config, seed)
        self.ds = W.device_values(self.spec, self.meta, seed=seed)
        self.out = torch.empty_like(self.ds.q)
        m = self.meta
        self.ws = B.alloc_workspace(m.num_seqs, m.total_q, m.max_seqlen_k, self.spec.num_heads,
                                    self.spec.head_dim)
        self.launch, self.entry, self.stream = launch, entry, stream
        self.one_call = entry == "step" and launch == "fused"

    def attention(self):
        B, ds, m = self.B, self.ds, self.meta
        if self.launch == "fused":
            B.hybrid_attn_fwd(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q, ds.seqlens_k,
                              ds.block_table, m.max_seqlen_q, m.max_seqlen_k, out=self.out,
                              workspace=self.ws, stream=self.stream)
        else:
            B.hybrid_attn_fwd_two_launch(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q,
                                         ds.seqlens_k, ds.block_table, m.max_seqlen_q,
                                         m.max_seqlen_k, out=self.out, workspace=self.ws,
                                         two_streams=self.launch == "two-streams",
                                         stream=self.stream)

    def append(self):
        ds = self.ds
        self.B.paged_kv_append(ds.key, ds.value, ds.slot_mapping, ds.k_cache, ds.v_cache,
                               stream=self.stream)

    def step(self):
        B, ds, m = self.B, self.ds, self.meta
        if self.one_call:
            B.hybrid_step_fwd(ds.key, ds.value, ds.slot_mapping, ds.q, ds.k_cache, ds.v_cache,
                              ds.cu_seqlens_q, ds.seqlens_k, ds.block_table, m.max_seqlen_q,
                              m.max_seqlen_k, out=self.out, workspace=self.ws, stream=self.stream)
            return
        self.append()
        self.attention()

    def free(self):
        del self.ds, self.out, self.ws
        import gc
        gc.collect()
        self.torch.cuda.empty_cache()


class Flush:
    """Cache eviction before a timed step, on the step's stream.  "read" sums a
    1 GiB buffer into one float: every XCD's L2 and the MALL are refilled with
    the buffer, so the step meets its inputs in HBM, and nothing dirty is left
    behind.  "write" fills a 1 GiB buffer: the same eviction, but it leaves up
    to the MALL's and the L2s' capacity of dirty lines, whose write-back to HBM
    then runs during the timed step and is charged to it."""

    def __init__(self, torch, kind):
        self.torch, self.kind = torch, kind
        if kind == "read":
            self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
            self.acc = torch.zeros((), dtype=torch.float32, device="cuda")
        else:
            self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def __call__(self, stream):
        with self.torch.cuda.stream(stream):
            if self.kind == "read":
                self.torch.sum(self.buf, dim=(0,), out=self.acc)
            else:
                self.buf.fill_(1)


def timed_steps(r: Runner, steps, flush):
    """Per-step durations (ms, HIP events on r.stream) of `steps` steps, each
    preceded by flush(r.stream) when a flush is given; and the wall time of
    the whole loop, bracketed by device synchronisation."""
    torch = r.torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        if flush is not None:
            flush(r.stream)
        e0.record(r.stream)
        r.step()
        e1.record(r.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return np.array([e0.elapsed_time(e1) for e0, e1 in ev]), wall


def timed_calls(r: Runner, steps, flush):
    """Durations (ms) of the append and of the attention call, as two
    separate calls per step (each step preceded by the flush when given)."""
    torch = r.torch
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    for e0, e1, e2 in ev:
        if flush is not None:
            flush(r.stream)
        e0.record(r.stream)
        r.append()
        e1.record(r.stream)
        r.attention()
        e2.record(r.stream)
    torch.cuda.synchronize()
    return (np.array([e0.elapsed_time(e1) for e0, e1, _ in ev]),
            np.array([e1.elapsed_time(e2) for _, e1, e2 in ev]))


def percentiles(ms):
    """p10 / p50 / p90 of per-step durations given in ms, in us."""
    return {f"p{q}": round(float(np.percentile(ms, q)) * 1e3, 2) for q in (10, 50, 90)}


def measure(r: Runner, steps, warmup, flushes):
    """flushes: {"read": Flush, "write": Flush}, or None for no flush at all."""
    torch = r.torch
    with torch.cuda.stream(r.stream):
        for _ in range(warmup):
            r.step()
    torch.cuda.synchronize()
    flush = flushes["read"] if flushes else None
    cold_ms, cold_wall = timed_steps(r, steps, flush)
    warm_ms, warm_wall = timed_steps(r, steps, None)
    append_ms, attn_ms = timed_calls(r, steps, flush)
    wflush_ms = timed_steps(r, steps, flushes["write"])[0] if flushes else None
    w = algorithmic_work(r.meta, r.spec)
    roof_us, bound = step_roofline_us(w, r.spec)
    cold_us = float(np.median(cold_ms)) * 1e3
    return {"w": w, "roof_us": roof_us, "bound": bound, "cold_ms": cold_ms, "cold_us": cold_us,
            "cold_wall": cold_wall, "warm_ms": warm_ms, "warm_wall": warm_wall,
            "append_ms": append_ms, "attn_ms": attn_ms, "wflush_ms": wflush_ms}


def write_flush_us(m):
    """Median step after the write flush (us), or None when no flush ran."""
    return None if m["wflush_ms"] is None else round(float(np.median(m["wflush_ms"])) * 1e3, 2)


def summary(r: Runner, m) -> dict:
    """Per-workload figures (the extra workloads' entry of the JSON line)."""
    attn_us = float(np.mean(m["attn_ms"])) * 1e3
    return {"cold_us_per_step": round(m["cold_us"], 2),
            "warm_us_per_step": round(1e3 * float(np.median(m["warm_ms"])), 2),
            "after_write_flush_us_per_step": write_flush_us(m),
            "step_roofline_us": round(m["roof_us"], 2), "bound": m["bound"],
            "frac_step_roofline": round(m["roof_us"] / m["cold_us"], 4),
            "attn_us": round(attn_us, 2),
            "append_us": round(float(np.mean(m["append_ms"])) * 1e3, 2)}


def main():
    from chunked_prefill_mixed_hybrid_amd import workload as W
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="4", choices=list(W.CONFIGS))
    ap.add_argument("--extra", default="1,2,3,5a,5b",
                    help="other workloads measured after the headline one (comma list, '' for none)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the 1 GiB cache flush before each timed step")
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

    B.load()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    flushes = None if args.no_flush else {"read": Flush(torch, "read"), "write": Flush(torch, "write")}

    r = Runner(args.config, args.seed, args.launch, args.entry, stream)
    spec, meta = r.spec, r.meta
    print(f"[bench] {spec.name}: {meta.num_seqs} segments, {meta.total_q} rows", file=sys.stderr,
          flush=True)
    m = measure(r, args.steps, args.warmup, flushes)
    w = m["w"]
    us_step = m["cold_us"]
    peak_tf = PEAK_MFMA_TFLOPS[spec.dtype]

    # roofline of the attention call (planner, attn_kernel, combine): its own
    # algorithmic bytes, or FLOPs when those bound it, over its mean duration
    attn_us = float(np.mean(m["attn_ms"])) * 1e3
    t_attn_hbm = w["attn_bytes"] / (PEAK_HBM_GBS * 1e9)
    t_attn_mfma = w["flops"] / (peak_tf * 1e12)
    if t_attn_hbm >= t_attn_mfma:
        achieved = w["attn_bytes"] / (attn_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        achieved = w["flops"] / (attn_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4), "traffic": None}
    if args.launch == "fused":
        roof["kernel"] = "hybrid_attn_fwd (plan_kernel + attn_kernel + combine_kernel, back to back)"
        roof["traffic"] = profiled_traffic(spec.name)
    else:
        roof["kernel"] = (f"hybrid_attn_fwd_two_launch ({args.launch}: plan, chunk launch, decode launch, "
                          "combine)")
    roof["avg_us"] = round(attn_us, 2)
    roof["algorithmic_bytes"] = w["attn_bytes"]
    roof["flush"] = not args.no_flush

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
                   "entry": "hybrid_step_fwd" if r.one_call else "paged_kv_append + attention",
                   "timing": ("median of per-step HIP events, each step after a 1 GiB read that "
                              "evicts L2 and the MALL" if flushes else
                              "median of per-step HIP events, no flush")},
        "timed_region_s": round(m["cold_wall"], 4),
        "warm_us_per_step": round(1e6 * m["warm_wall"] / args.steps, 2),
        "after_write_flush_us_per_step": write_flush_us(m),
        "tflops": round(w["flops"] / (us_step * 1e-6) / 1e12, 2),
        "kv_gbps": round(w["kv_bytes"] / (us_step * 1e-6) / 1e9, 1),
        "step_gbps": round(w["step_bytes"] / (us_step * 1e-6) / 1e9, 1),
        "step_roofline_us": round(m["roof_us"], 2),
        "step_roofline_bound": m["bound"],
        "frac_step_roofline": round(m["roof_us"] / us_step, 4),
        "frac_step_roofline_warm": round(m["roof_us"] / (1e6 * m["warm_wall"] / args.steps), 4),
        "append_us": round(float(np.mean(m["append_ms"])) * 1e3, 2),
        "attn_us": round(attn_us, 2),
        "step_us_percentiles": percentiles(m["cold_ms"]),
        "warm_us_percentiles": percentiles(m["warm_ms"]),
        "roofline": roof,
    }
    if args.calibrate_copy:  # a copy of known size: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(r.ds, spec, meta, w)
    r.free()
    extras = {}
    for c in [c for c in args.extra.split(",") if c and c != args.config]:
        rx = Runner(c, args.seed, args.launch, args.entry, stream)
        print(f"[bench] extra workload {rx.spec.name}", file=sys.stderr, flush=True)
        extras[rx.spec.name] = summary(rx, measure(rx, args.steps, args.warmup, flushes))
        rx.free()
    if extras:
        result["workloads"] = extras
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
