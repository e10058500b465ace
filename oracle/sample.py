"""Copies some segments of a step out of device memory for the oracle.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
baseline leg).  A step of the long-context or decode-heavy workload holds
70-75 GB of pages; the oracle checks it a few segments at a time.  This module
gathers, for a chosen set of segments, their pages (block ids renumbered
compactly), query rows, new keys and values and metadata into host arrays.
It holds none of the attention arithmetic: the oracle does that.
"""
from __future__ import annotations

import numpy as np

from .oracle import default


def host_array(t) -> np.ndarray:
    """torch tensor (any device) -> numpy; bf16 becomes its raw uint16 bits."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class SampledStep:
    """Pages, rows and metadata of some segments of a step whose tensors live
    on the device.  Built BEFORE the device append, so the oracle's own append
    runs on the same pre-append bytes.

    meta: host metadata (cu_seqlens_q, seqlens_k, block_table, slot_mapping,
    page_size); q, key, value, k_cache, v_cache: device tensors."""

    def __init__(self, meta, q, key, value, k_cache, v_cache, segs):
        import torch
        p = meta.page_size
        self.segs = list(segs)
        pages, rows, lqs, lks = [], [], [], []
        for b in self.segs:
            lk = int(meta.seqlens_k[b])
            r0, r1 = int(meta.cu_seqlens_q[b]), int(meta.cu_seqlens_q[b + 1])
            n = (lk + p - 1) // p
            pages.append(meta.block_table[b, :n].astype(np.int64))
            rows.append(np.arange(r0, r1))
            lqs.append(r1 - r0)
            lks.append(lk)
        allp = np.concatenate(pages)
        self.pages = allp
        self.rows = np.concatenate(rows)
        remap = {int(pg): i for i, pg in enumerate(allp)}
        mb = max(1, max(len(x) for x in pages))
        bt = np.full((len(self.segs), mb), -1, np.int32)
        off = 0
        for i, x in enumerate(pages):
            bt[i, :len(x)] = np.arange(off, off + len(x))
            off += len(x)
        self.block_table = bt
        self.cu = np.concatenate([[0], np.cumsum(lqs)]).astype(np.int32)
        self.sk = np.array(lks, np.int32)
        slots = meta.slot_mapping[self.rows].astype(np.int64)
        self.slot_mapping = np.array([remap[int(s) // p] * p + int(s) % p for s in slots], np.int32)
        idx = torch.from_numpy(allp).to(k_cache.device)
        self.kc = host_array(k_cache.index_select(0, idx))
        self.vc = host_array(v_cache.index_select(0, idx))
        ridx = torch.from_numpy(self.rows).to(q.device)
        self.q = host_array(q.index_select(0, ridx))
        self.key = host_array(key.index_select(0, ridx))
        self.value = host_array(value.index_select(0, ridx))
        self.page_idx = idx

    @property
    def nbytes(self) -> int:
        return self.kc.nbytes + self.vc.nbytes

    def oracle(self, row_select=None, orc=None):
        """Oracle append, then attention, on these segments: (out, k pages, v pages)."""
        orc = orc or default()
        kc, vc = self.kc.copy(), self.vc.copy()
        orc.append(self.key, self.value, self.slot_mapping, kc, vc)
        out = orc.attention(self.q, kc, vc, self.cu, self.sk, self.block_table,
                            row_select=row_select)
        return out, kc, vc


def segment_batches(meta, segs, max_bytes, bytes_per_key):
    """Consecutive groups of `segs` whose pages (both pools) stay within
    max_bytes of host memory each (a segment larger than that is a group of
    its own)."""
    out, cur, cur_b = [], [], 0
    p = meta.page_size
    for b in segs:
        nb = 2 * ((int(meta.seqlens_k[b]) + p - 1) // p) * p * bytes_per_key
        if cur and cur_b + nb > max_bytes:
            out.append(cur)
            cur, cur_b = [], 0
        cur.append(int(b))
        cur_b += nb
    if cur:
        out.append(cur)
    return out
