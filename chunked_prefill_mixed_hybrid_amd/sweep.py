"""Tile-quantisation sweep: time of one mixed step as a function of the chunk
length around multiples of the chunk tile (128 query rows).

A token budget that overshoots a tile multiple by one token buys a whole extra
query tile per head: the wangyu.me chunked-prefill page (section on how large
the chunk should be) relays a measurement with 128-wide tiles where 257 tokens
took about a third longer than 256, which is why step budgets get aligned to
tile boundaries.  This sweep measures that effect for the fused kernel on MI355X: one
chunk of length L at history H0, alone or packed with 30 decode segments of the
bench workload's shape, 32 heads x 128, bf16, 16-token pages.

    python -m chunked_prefill_mixed_hybrid_amd.sweep [--history 1536] [--reps 50]
    python -m chunked_prefill_mixed_hybrid_amd.sweep trace
    python -m chunked_prefill_mixed_hybrid_amd.sweep kv

The first prints one JSON line per (L, decodes) point and a table; `trace`
runs a 64-request trace through the token-budget step generator (one JSON
line: steps, tokens/s, per-step times, fraction of the per-step rooflines);
`kv` times the attention call on paged K/V and on the same keys packed per
segment (varlen_attn_fwd).
Synthetic inputs (seeded), as everywhere in this package.
"""
from __future__ import annotations

import argparse
import json

import numpy as np

DEFAULT_LENGTHS = (896, 960, 1023, 1024, 1025, 1056, 1088, 1151, 1152, 1153, 1280)


def _decodes(n: int, seed: int):
    rng = np.random.default_rng(seed)
    hist = rng.integers(512, 4096, n, endpoint=True)
    return [(1, int(h) + 1) for h in hist]


def time_step(segments, heads=32, head_dim=128, reps=50, warmup=5, seed=0):
    """Median microseconds of hybrid_attn_fwd over `reps` calls (HIP events on
    the stream the kernels run on) for one step of the given segments."""
    import torch
    from . import binding as B
    from . import workload as W
    spec, meta = W.custom_step(segments, heads, heads, head_dim, W.BF16, seed=seed)
    ds = W.device_values(spec, meta, seed=seed)
    out = torch.empty_like(ds.q)
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, heads, head_dim)
    stream = torch.cuda.current_stream()

    def call():
        B.hybrid_attn_fwd(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q, ds.seqlens_k,
                          ds.block_table, meta.max_seqlen_q, meta.max_seqlen_k, out=out,
                          workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in times]) * 1e3)
    del ds, out, ws
    torch.cuda.empty_cache()
    return us


def trace(num_requests=64, budget=2048, threshold=0, prompt=(256, 4096), new_tokens=(16, 128),
          heads=32, head_dim=128, seed=0):
    """A request trace scheduled by the token-budget step generator and run step
    by step (paged_kv_append + hybrid_attn_fwd on one page pool): per-step GPU
    time (HIP events, scheduling and metadata uploads outside), tokens and
    algorithmic bytes.  Values are random; every request arrives at the start."""
    import torch
    from . import binding as B
    from .scheduler import StepScheduler
    rng = np.random.default_rng(seed)
    plens = rng.integers(prompt[0], prompt[1], num_requests, endpoint=True)
    gens = rng.integers(new_tokens[0], new_tokens[1], num_requests, endpoint=True)
    page = 16
    nb = int(sum(-(-int(p + g) // page) for p, g in zip(plens, gens))) + 64
    mb = int(max(-(-int(p + g) // page) for p, g in zip(plens, gens)))
    s = StepScheduler(budget, nb, mb, long_prefill_token_threshold=threshold,
                      max_seqs=num_requests)
    for r, (p, g) in enumerate(zip(plens, gens)):
        s.add(r, int(p), int(g))
    kc = torch.zeros((nb, page, heads, head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ws = B.alloc_workspace(num_requests, budget, mb * page, heads, head_dim)
    stream = torch.cuda.current_stream()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()  # noqa: E731
    steps = []
    while (st := s.next_step()) is not None:
        t = st.total_q
        q = torch.randn((t, heads, head_dim), device="cuda").to(torch.bfloat16)
        k = torch.randn((t, heads, head_dim), device="cuda").to(torch.bfloat16)
        v = torch.randn((t, heads, head_dim), device="cuda").to(torch.bfloat16)
        sm, cu, sk, bt = i32(st.slot_mapping), i32(st.cu_seqlens_q), i32(st.seqlens_k), i32(st.block_table)
        out = torch.empty_like(q)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        B.paged_kv_append(k, v, sm, kc, vc, stream=stream)
        B.hybrid_attn_fwd(q, kc, vc, cu, sk, bt, st.max_seqlen_q, st.max_seqlen_k, out=out,
                          workspace=ws, stream=stream)
        e1.record(stream)
        lq = np.diff(st.cu_seqlens_q).astype(np.int64)
        lk = st.seqlens_k.astype(np.int64)
        kv_bytes = 2.0 * head_dim * heads * 2 * float(lk.sum())
        bytes_ = kv_bytes + 2.0 * head_dim * heads * (2 + 4) * t + 4.0 * (
            float(((lk + 15) // 16).sum()) + 2 * len(lk) + 1 + t)
        vis = lq * (lk - lq) + lq * (lq + 1) // 2
        flops = 4.0 * head_dim * heads * float(vis.sum())
        steps.append((e0, e1, t, st.num_seqs, st.num_decodes, bytes_, flops))
        s.complete()
    torch.cuda.synchronize()
    rows = []
    for e0, e1, t, b, nd, by, fl in steps:
        us = e0.elapsed_time(e1) * 1e3
        roof = max(by / 8e12, fl / 2.5e15) * 1e6
        rows.append((us, t, b, nd, roof))
    a = np.array(rows)
    res = {"requests": num_requests, "budget": budget, "steps": len(rows),
           "tokens": int(a[:, 1].sum()), "gpu_ms": round(float(a[:, 0].sum()) / 1e3, 2),
           "tokens_per_s": round(float(a[:, 1].sum() / (a[:, 0].sum() * 1e-6)), 1),
           "us_per_step_median": round(float(np.median(a[:, 0])), 1),
           "us_per_step_p90": round(float(np.percentile(a[:, 0], 90)), 1),
           "frac_of_step_rooflines": round(float(a[:, 4].sum() / a[:, 0].sum()), 4),
           "mixed_steps": int(((a[:, 3] > 0) & (a[:, 3] < a[:, 2])).sum()),
           "decode_only_steps": int((a[:, 3] == a[:, 2]).sum())}
    return res


def kv_layouts(configs=(2, 5, 1), reps=30):
    """Attention-call time on paged K/V (hybrid_attn_fwd) and on the same keys
    packed per segment (varlen_attn_fwd), per workload config."""
    import torch
    from . import binding as B
    from . import workload as W
    res = []
    for c in configs:
        spec, meta = W.make_step(c)
        ds = W.device_values(spec, meta, seed=0) if spec.dtype == W.BF16 else \
            W.to_device(W.host_values(spec, meta, seed=0))
        B.paged_kv_append(ds.key, ds.value, ds.slot_mapping, ds.k_cache, ds.v_cache)
        slots = []
        for b, lk in enumerate(meta.seqlens_k.tolist()):
            j = np.arange(lk)
            slots.append(meta.block_table[b, j // meta.page_size] * meta.page_size + j % meta.page_size)
        idx = torch.from_numpy(np.concatenate(slots).astype(np.int64)).cuda()
        nb, pg, hkv, d = ds.k_cache.shape
        k = ds.k_cache.reshape(nb * pg, hkv, d).index_select(0, idx)
        v = ds.v_cache.reshape(nb * pg, hkv, d).index_select(0, idx)
        cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(meta.seqlens_k)]).astype(np.int32)).cuda()
        out = torch.empty_like(ds.q)
        ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, spec.num_heads,
                               spec.head_dim)
        calls = {
            "paged": lambda: B.hybrid_attn_fwd(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q,
                                               ds.seqlens_k, ds.block_table, meta.max_seqlen_q,
                                               meta.max_seqlen_k, out=out, workspace=ws),
            "contiguous": lambda: B.varlen_attn_fwd(ds.q, k, v, ds.cu_seqlens_q, cu_k,
                                                    meta.max_seqlen_q, meta.max_seqlen_k,
                                                    out=out, workspace=ws)}
        row = {"workload": spec.name}
        for name, f in calls.items():
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            row[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
        res.append(row)
        print(json.dumps(row), flush=True)
        del ds, k, v, out, ws
        torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("mode", nargs="?", default="tiles", choices=["tiles", "trace", "kv"])
    ap.add_argument("--lengths", default=",".join(map(str, DEFAULT_LENGTHS)))
    ap.add_argument("--history", type=int, default=1536, help="chunk history H0 (keys before it)")
    ap.add_argument("--decodes", default="0,30", help="decode segments packed with the chunk")
    ap.add_argument("--reps", type=int, default=50)
    args = ap.parse_args(argv)
    from . import binding as B
    B.load()  # fail loudly if the HIP library is missing
    if args.mode == "trace":
        print(json.dumps(trace()), flush=True)
        return
    if args.mode == "kv":
        kv_layouts()
        return
    rows = []
    for nd in (int(x) for x in args.decodes.split(",")):
        dec = _decodes(nd, seed=1)
        for L in (int(x) for x in args.lengths.split(",")):
            segs = [(L, args.history + L)] + dec
            us = time_step(segs, reps=args.reps)
            tiles = -(-L // 128)
            row = {"chunk_len": L, "history": args.history, "decodes": nd, "tiles_per_head": tiles,
                   "us": round(us, 2), "us_per_token": round(us / (L + nd), 4)}
            rows.append(row)
            print(json.dumps(row), flush=True)
    print(f"{'decodes':>7} {'L':>6} {'tiles':>5} {'us':>9} {'us/token':>9}")
    for r in rows:
        print(f"{r['decodes']:>7} {r['chunk_len']:>6} {r['tiles_per_head']:>5} {r['us']:>9.2f} "
              f"{r['us_per_token']:>9.4f}")


if __name__ == "__main__":
    main()
