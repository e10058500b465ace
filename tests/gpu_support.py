"""Helpers of the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same bytes, compare at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

from chunked_prefill_mixed_hybrid_amd import binding as B
from chunked_prefill_mixed_hybrid_amd import workload as W
import oracle as O
from oracle import sample as OS

# Tolerances: fp32 max |err| <= 1e-4; bf16 max |err| <= 2e-2 AND
# ||err||_2 / ||ref||_2 <= 1e-2 (both must hold); any NaN/Inf fails.
TOL_F32_ABS = 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 1e-2


def note(msg: str) -> None:
    """Progress line that bypasses pytest capture (names the GPU case first)."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a GPU")
    B.load()


def gpu_step(ds: W.DeviceStep, workspace=None, append=True):
    """paged_kv_append then hybrid_attn_fwd, exactly as a step runs them."""
    import torch
    m = ds.meta
    if append:
        B.paged_kv_append(ds.key, ds.value, ds.slot_mapping, ds.k_cache, ds.v_cache)
    out = torch.empty_like(ds.q)
    B.hybrid_attn_fwd(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q, ds.seqlens_k,
                      ds.block_table, m.max_seqlen_q, m.max_seqlen_k, out=out,
                      workspace=workspace)
    torch.cuda.synchronize()
    return out


PLAN_HEADER_FIELDS = ("dec_counter", "n_chunk_tiles", "n_dec_items", "n_dec_full", "split",
                      "n_parts", "bad_segments", "chunk_split")


def plan_header(workspace) -> dict:
    """The planner's summary of the last call, read from the workspace head
    (8 chunk-group counters, then the int32 fields above, in order)."""
    raw = workspace[:64].cpu().numpy().view(np.int32)
    return dict(zip(PLAN_HEADER_FIELDS, (int(v) for v in raw[8:8 + len(PLAN_HEADER_FIELDS)])))


def contiguous_kv(ds: W.DeviceStep, poison_rows: int = 5):
    """Each segment's logical keys and values gathered out of the (appended)
    paged pools into packed [total_k, Hkv, D] buffers, followed by NaN rows, and
    the matching cu_seqlens_k -- the same data in the varlen contiguous layout."""
    import torch
    m = ds.meta
    slots = []
    for b, lk in enumerate(m.seqlens_k.tolist()):
        j = np.arange(lk)
        slots.append(m.block_table[b, j // m.page_size] * m.page_size + j % m.page_size)
    idx = torch.from_numpy(np.concatenate(slots).astype(np.int64)).to(ds.k_cache.device)
    nb, p, hkv, d = ds.k_cache.shape
    k = ds.k_cache.reshape(nb * p, hkv, d).index_select(0, idx)
    v = ds.v_cache.reshape(nb * p, hkv, d).index_select(0, idx)
    pad = torch.full((poison_rows, hkv, d), float("nan"), dtype=k.dtype, device=k.device)
    cu_k = np.concatenate([[0], np.cumsum(m.seqlens_k)]).astype(np.int32)
    return (torch.cat([k, pad]).contiguous(), torch.cat([v, pad]).contiguous(),
            torch.from_numpy(cu_k).to(k.device))


def equal_device(a, b, slab=1 << 29) -> bool:
    """Bitwise equality of two device tensors, compared in slabs of raw bytes."""
    import torch
    fa, fb = a.reshape(-1).view(torch.uint8), b.reshape(-1).view(torch.uint8)
    if fa.numel() != fb.numel():
        return False
    return all(torch.equal(fa[s:s + slab], fb[s:s + slab]) for s in range(0, fa.numel(), slab))


def to_f64(t) -> np.ndarray:
    return O.to_f64(W.to_host_array(t))


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """got, ref: float64 arrays of the same shape."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - ref
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(err) / nref) if nref > 0 else 0.0
    stats = {"max_abs": max_abs, "rel_norm": rel}
    if dtype == W.F32:
        assert max_abs <= TOL_F32_ABS, f"{what}: fp32 max abs err {max_abs}"
    else:
        assert max_abs <= TOL_BF16_ABS, f"{what}: bf16 max abs err {max_abs}"
        assert rel <= TOL_BF16_REL, f"{what}: bf16 rel norm err {rel}"
    return stats


def host_pools(ds: W.DeviceStep):
    return W.to_host_array(ds.k_cache), W.to_host_array(ds.v_cache)


def oracle_full(ds: W.DeviceStep, kc_host, vc_host, row_select=None):
    """Oracle append + attention on host copies of the PRE-append pools."""
    orc = O.default()
    m = ds.meta
    kc, vc = kc_host.copy(), vc_host.copy()
    orc.append(W.to_host_array(ds.key), W.to_host_array(ds.value), m.slot_mapping, kc, vc)
    out = orc.attention(W.to_host_array(ds.q), kc, vc, m.cu_seqlens_q, m.seqlens_k,
                        m.block_table, row_select=row_select)
    return out, kc, vc


def sampled_step(ds: W.DeviceStep, segs) -> OS.SampledStep:
    """Host copies of the pages, rows and metadata of segments `segs` of a
    device step (taken before its append), for the oracle."""
    return OS.SampledStep(ds.meta, ds.q, ds.key, ds.value, ds.k_cache, ds.v_cache, segs)
