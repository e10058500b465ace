"""Dense brute-force attention for tiny inputs (TEST INFRASTRUCTURE ONLY).

Works on LOGICAL, unpaged K/V (one [Lk, Hkv, D] array per segment), builds the
full score matrix with an explicit mask matrix M[i, j] = (j <= Lk - Lq + i)
(query segment right-aligned to its KV segment, as on the wangyu.me Chunked
Prefill page, section "Flash Attention 的 varlen 接口"), applies a row softmax
and multiplies by V.  numpy matmul is the only library primitive used.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def mask_matrix(lq: int, lk: int) -> np.ndarray:
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= (lk - lq) + i


def dense_attention(q: np.ndarray, seg_k: list, seg_v: list, cu_seqlens_q,
                    scale: float | None = None) -> np.ndarray:
    """q [T, Hq, D]; seg_k[b], seg_v[b]: [Lk_b, Hkv, D] logical keys/values."""
    q = to_f64(q)
    t, hq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((t, hq, d))
    for b in range(len(seg_k)):
        r0, r1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        if r1 == r0:
            continue
        k = to_f64(seg_k[b])
        v = to_f64(seg_v[b])
        lk, hkv, _ = k.shape
        group = hq // hkv
        m = mask_matrix(r1 - r0, lk)
        for h in range(hq):
            s = scale * (q[r0:r1, h, :] @ k[:, h // group, :].T)
            s = np.where(m, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w = w / w.sum(axis=1, keepdims=True)
            out[r0:r1, h, :] = w @ v[:, h // group, :]
    return out
