"""hybrid_step_fwd_noalloc (the library's own device scratch array as the
workspace, no allocation in the call) against hybrid_step_fwd with a
caller-allocated workspace, through the C ABI: four calls in a row on
shrinking inputs.  Pools byte-identical; outputs within the oracle's bf16 /
fp32 tolerance of the workspace call's, and byte-identical where that call's
workspace fits the 64 MiB array (same plan, same kernels)."""
import numpy as np
import pytest

from chunked_prefill_mixed_hybrid_amd import binding as B
from chunked_prefill_mixed_hybrid_amd import workload as W
import gpu_support as G

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _steps():
    """(name, spec, meta, host step or None): a one-segment bf16 prefill (the
    path that uses no workspace), the mixed workload (its usual workspace is
    larger than the scratch array: capped layout), the worked example (fp32,
    split chunk tiles: chunk partials in the array), a small step."""
    spec0, meta0 = W.custom_step([(1000, 1500)], 64, 64, 128, W.BF16, seed=6)
    spec2, meta2 = W.make_step(2)
    spec1, meta1 = W.make_step(1)
    spec3, meta3 = W.custom_step([(1, 300), (70, 500), (1, 40)], 4, 4, 128, W.BF16, seed=5)
    return [("one-segment prefill", spec0, meta0, None), ("mixed", spec2, meta2, None),
            ("worked example", spec1, meta1, W.host_values(spec1, meta1)),
            ("small", spec3, meta3, W.host_values(spec3, meta3, seed=5))]


def _workspace_call(ds):
    import torch
    m = ds.meta
    out = torch.empty_like(ds.q)
    ws = B.alloc_workspace(m.num_seqs, m.total_q, m.max_seqlen_k, ds.spec.num_heads, ds.spec.head_dim)
    B.hybrid_step_fwd(ds.key, ds.value, ds.slot_mapping, ds.q, ds.k_cache, ds.v_cache,
                      ds.cu_seqlens_q, ds.seqlens_k, ds.block_table, m.max_seqlen_q, m.max_seqlen_k,
                      out=out, workspace=ws)
    torch.cuda.synchronize()
    return out, ws.numel()


def test_noalloc_matches_workspace_entry():
    import torch
    G.require_gpu()
    sizes = []
    for name, spec, meta, hs in _steps():
        G.note(f"noalloc: {name} ({meta.num_seqs} segments, {meta.total_q} rows, {spec.dtype})")
        if hs is None:
            ds_a = W.device_values(spec, meta, seed=0)
            ds_b = W.DeviceStep(spec, meta, ds_a.q, ds_a.key, ds_a.value, ds_a.k_cache.clone(),
                                ds_a.v_cache.clone(), ds_a.cu_seqlens_q, ds_a.seqlens_k,
                                ds_a.block_table, ds_a.slot_mapping)
        else:
            ds_a, ds_b = W.to_device(hs, "cuda"), W.to_device(hs, "cuda")
        sizes.append(ds_a.q.numel() * ds_a.q.element_size())
        ref, ws_bytes = _workspace_call(ds_a)
        out = torch.full_like(ds_b.q, float("nan"))
        m = ds_b.meta
        B.hybrid_step_fwd_noalloc(ds_b.key, ds_b.value, ds_b.slot_mapping, ds_b.q, ds_b.k_cache,
                                  ds_b.v_cache, ds_b.cu_seqlens_q, ds_b.seqlens_k, ds_b.block_table,
                                  m.max_seqlen_q, m.max_seqlen_k, out)
        torch.cuda.synchronize()
        assert G.equal_device(ds_a.k_cache, ds_b.k_cache) and G.equal_device(ds_a.v_cache, ds_b.v_cache)
        G.compare(G.to_f64(out), G.to_f64(ref), spec.dtype, f"noalloc {name}")
        if ws_bytes <= SCRATCH_BYTES:
            assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), name
        del ds_a, ds_b, ref, out
    assert sizes == sorted(sizes, reverse=True)  # each call's input smaller than the last
