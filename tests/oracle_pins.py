"""Pins of the CPU oracle against facts the source pages and mathematics fix.

Every pin takes an `Oracle` instance so the same checks run against the real
oracle and against deliberately broken copies (test_oracle_mutants.py): each
planted mistake must make at least one pin fail.

Sources of the facts:
  * worked example and right-aligned causal visibility: "大语言模型推理优化（二）：
    Chunked Prefill" (wangyu.me), sections "记录 KV Cache 的长度" and
    "Flash Attention 的 varlen 接口";
  * chunking does not change results: same page, section "Chunked Prefill 的注意力计算";
  * decode == a length-1 segment, unmasked: same page, end of the varlen section;
  * page translation: kwkr.cn Triton article, kernel section (block table row,
    pos // PAGE_SIZE, pos % PAGE_SIZE);
  * append through slot_mapping before attention: wangyu.me page, section
    "输入组装".
"""
from __future__ import annotations

import json
from fractions import Fraction
from pathlib import Path

import numpy as np

from chunked_prefill_mixed_hybrid_amd import workload as W
import oracle as O

GOLDEN = Path(__file__).resolve().parent / "golden"


def golden(name):
    return json.loads((GOLDEN / name).read_text())


def run_step(orc, hs: W.HostStep, row_select=None):
    """Append this step's K/V (on copies of the pools), then attend."""
    kc, vc = hs.k_cache.copy(), hs.v_cache.copy()
    orc.append(hs.key, hs.value, hs.meta.slot_mapping, kc, vc)
    out = orc.attention(hs.q, kc, vc, hs.meta.cu_seqlens_q, hs.meta.seqlens_k,
                        hs.meta.block_table, row_select=row_select)
    return out, kc, vc


def logical_kv(hs: W.HostStep):
    """Per segment, the logical [Lk, Hkv, D] keys/values: history read from the
    pool at the slot each position was given by the metadata builder, then this
    step's new tokens straight from key/value (no append involved)."""
    m, p = hs.meta, hs.meta.page_size
    hkv, d = hs.spec.num_kv_heads, hs.spec.head_dim
    kflat = hs.k_cache.reshape(-1, hkv, d)
    vflat = hs.v_cache.reshape(-1, hkv, d)
    ks, vs = [], []
    for b in range(m.num_seqs):
        r0, r1 = int(m.cu_seqlens_q[b]), int(m.cu_seqlens_q[b + 1])
        lk = int(m.seqlens_k[b])
        h0 = lk - (r1 - r0)
        pos = np.arange(h0)
        slots = m.block_table[b, pos // p].astype(np.int64) * p + pos % p
        ks.append(np.concatenate([kflat[slots], hs.key[r0:r1]]))
        vs.append(np.concatenate([vflat[slots], hs.value[r0:r1]]))
    return ks, vs


# ------------------------------------------------------------------------ P1
def pin_worked_example_metadata(orc):
    g = golden("worked_example.json")
    spec, meta = W.make_step(1)
    assert meta.cu_seqlens_q.tolist() == g["cu_seqlens_q"]
    cu_k = np.concatenate([[0], np.cumsum(meta.seqlens_k)]).tolist()
    assert cu_k == g["cu_seqlens_k"]
    assert meta.max_seqlen_q == g["max_seqlen_q"] and meta.max_seqlen_k == g["max_seqlen_k"]
    reqs = g["requests"]
    assert [lk for _, lk in spec.segments] == [r["history"] + r["new_tokens"] for r in reqs]
    assert orc.check_slots(meta.cu_seqlens_q, meta.seqlens_k, meta.block_table,
                           meta.slot_mapping, meta.page_size, meta.num_blocks) == 0
    gp = golden("mixed_packing.json")
    segs = [(lq, lq + 100) for lq in gp["query_lengths"]]
    _, m2 = W.custom_step(segs, 1, 1, 8, W.F32)
    assert m2.cu_seqlens_q.tolist() == gp["cu_seqlens"]


def pin_worked_example_visibility(orc):
    g = golden("worked_example.json")
    n = orc.visible_counts(g["cu_seqlens_q"], np.diff(g["cu_seqlens_k"]))
    assert n[0] == g["visible_keys"]["A"] and n[1] == g["visible_keys"]["B"]
    hist_c = g["requests"][2]["history"]
    assert np.array_equal(n[2:], hist_c + np.arange(1808) + 1)
    assert n[2] == 8193 and n[-1] == 10000


def pin_worked_example_perturbation(orc, rows=(0, 1, 2, 3, 700, 1808, 1809)):
    """Changing the first invisible key of a row leaves it bitwise unchanged;
    changing its last visible key changes it."""
    spec, meta = W.make_step(1)
    hs = W.host_values(spec, meta, seed=0)
    sel = np.zeros(meta.total_q, np.uint8)
    sel[list(rows)] = 1
    base, kc, vc = run_step(orc, hs, sel)
    n_vis = orc.visible_counts(meta.cu_seqlens_q, meta.seqlens_k)
    p, hkv, d = meta.page_size, spec.num_kv_heads, spec.head_dim
    for r in rows:
        b = int(np.searchsorted(meta.cu_seqlens_q, r, side="right") - 1)
        for pos, must_change in ((int(n_vis[r]), False), (int(n_vis[r]) - 1, True)):
            if pos >= meta.seqlens_k[b]:
                continue
            slot = int(meta.block_table[b, pos // p]) * p + pos % p
            for cache in ("k", "v"):
                kc2, vc2 = kc.copy(), vc.copy()
                tgt = kc2 if cache == "k" else vc2
                tgt.reshape(-1, hkv, d)[slot] += 1.0
                one = np.zeros(meta.total_q, np.uint8)
                one[r] = 1
                out = orc.attention(hs.q, kc2, vc2, meta.cu_seqlens_q, meta.seqlens_k,
                                    meta.block_table, row_select=one)
                same = np.array_equal(out[r], base[r])
                assert same != must_change, (r, pos, cache, must_change)


# ------------------------------------------------------------------------ P2
def pin_chunk_invariance(orc, prompt=10000, chunk=2048, heads=1, d=8, dtype=W.BF16):
    """A prompt prefilled chunk by chunk gives the same output rows (bitwise,
    fp64) and the same cache bytes as one full prefill."""
    steps = W.chunked_prompt_steps(prompt, chunk)
    assert steps[:4] == [(2048, 2048), (2048, 4096), (2048, 6144), (2048, 8192)]
    assert steps[-1] == (1808, 10000) or prompt != 10000
    spec_full, meta_full = W.custom_step([(prompt, prompt)], heads, heads, d, dtype, seed=3,
                                         spare_blocks=4)
    hs_full = W.host_values(spec_full, meta_full, seed=3)
    out_full, kc_full, vc_full = run_step(orc, hs_full)

    kc, vc = hs_full.k_cache.copy(), hs_full.v_cache.copy()
    outs = []
    for lq, lk in steps:
        h0 = lk - lq
        cu = np.array([0, lq], np.int32)
        sk = np.array([lk], np.int32)
        sl = meta_full.slot_mapping[h0:lk]
        orc.append(hs_full.key[h0:lk], hs_full.value[h0:lk], sl, kc, vc)
        outs.append(orc.attention(np.ascontiguousarray(hs_full.q[h0:lk]), kc, vc, cu, sk,
                                  meta_full.block_table))
    assert np.array_equal(np.concatenate(outs), out_full)
    assert kc.tobytes() == kc_full.tobytes() and vc.tobytes() == vc_full.tobytes()


# ------------------------------------------------------------------------ P3
def pin_textbook_causal(orc):
    """Lq == Lk (no history): plain causal attention (torch SDPA, is_causal)."""
    import torch
    for dtype in (W.F32, W.BF16):
        spec, meta = W.custom_step([(37, 37), (16, 16), (1, 1)], 3, 3, 16, dtype, seed=5)
        hs = W.host_values(spec, meta, seed=5)
        out, _, _ = run_step(orc, hs)
        for b in range(meta.num_seqs):
            r0, r1 = meta.cu_seqlens_q[b], meta.cu_seqlens_q[b + 1]
            q = torch.from_numpy(O.to_f64(hs.q[r0:r1])).transpose(0, 1)
            k = torch.from_numpy(O.to_f64(hs.key[r0:r1])).transpose(0, 1)
            v = torch.from_numpy(O.to_f64(hs.value[r0:r1])).transpose(0, 1)
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
            assert np.max(np.abs(ref.transpose(0, 1).numpy() - out[r0:r1])) < 1e-12


def pin_decode_unmasked(orc):
    """Lq == 1: attention over all Lk keys with no mask (torch SDPA, no mask)."""
    import torch
    spec, meta = W.custom_step([(1, 1), (1, 16), (1, 17), (1, 100)], 2, 2, 32, W.F32, seed=6)
    hs = W.host_values(spec, meta, seed=6)
    out, _, _ = run_step(orc, hs)
    ks, vs = logical_kv(hs)
    for b in range(meta.num_seqs):
        r = meta.cu_seqlens_q[b]
        q = torch.from_numpy(O.to_f64(hs.q[r:r + 1])).transpose(0, 1)
        k = torch.from_numpy(O.to_f64(ks[b])).transpose(0, 1)
        v = torch.from_numpy(O.to_f64(vs[b])).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
        assert np.max(np.abs(ref.transpose(0, 1).numpy() - out[r:r + 1])) < 1e-12


def pin_prefix_means(orc):
    """q == 0: every visible key has the same score, so each row is the plain
    mean of its visible values (exact integer values, compared as fractions)."""
    segs = [(5, 40), (1, 3), (16, 16), (3, 50)]
    spec, meta = W.custom_step(segs, 2, 2, 8, W.F32, seed=7)
    hs = W.host_values(spec, meta, seed=7)
    hs.q[:] = 0
    rng = np.random.default_rng(7)
    hs.v_cache[:] = rng.integers(-50, 50, hs.v_cache.shape)
    hs.value[:] = rng.integers(-50, 50, hs.value.shape)
    out, _, _ = run_step(orc, hs)
    ks, vs = logical_kv(hs)
    for b, (lq, lk) in enumerate(segs):
        r0 = meta.cu_seqlens_q[b]
        csum = np.cumsum(vs[b].astype(np.int64), axis=0)
        for i in range(lq):
            n = lk - lq + i + 1
            exact = csum[n - 1] / n
            assert np.max(np.abs(out[r0 + i] - exact)) < 1e-12


def pin_single_key(orc):
    """Lk == 1: the output is exactly the only value row."""
    spec, meta = W.custom_step([(1, 1), (1, 1)], 2, 2, 16, W.BF16, seed=8)
    hs = W.host_values(spec, meta, seed=8)
    out, _, _ = run_step(orc, hs)
    assert np.array_equal(out, O.to_f64(hs.value))


def pin_constant_values_and_bounds(orc):
    """Constant V = c gives c; in general every output channel lies between the
    smallest and largest visible value of that channel."""
    segs = [(9, 70), (1, 33), (20, 20)]
    spec, meta = W.custom_step(segs, 2, 2, 16, W.F32, seed=9)
    hs = W.host_values(spec, meta, seed=9)
    out, _, _ = run_step(orc, hs)
    ks, vs = logical_kv(hs)
    for b, (lq, lk) in enumerate(segs):
        r0 = meta.cu_seqlens_q[b]
        v = vs[b].astype(np.float64)
        for i in range(lq):
            n = lk - lq + i + 1
            lo, hi = v[:n].min(axis=0), v[:n].max(axis=0)
            assert np.all(out[r0 + i] >= lo - 1e-12) and np.all(out[r0 + i] <= hi + 1e-12)
    hs.v_cache[:] = np.float32(0.375)
    hs.value[:] = np.float32(0.375)
    out, _, _ = run_step(orc, hs)
    assert np.max(np.abs(out - 0.375)) <= 4 * np.finfo(np.float64).eps


# ------------------------------------------------------------------------ P4
def brute_cases(quick=False):
    lqs = [1, 2, 15, 16, 17, 33]
    cases = []
    rng = np.random.default_rng(11)
    n_cases = 4 if quick else 12
    for c in range(n_cases):
        nseg = int(rng.integers(1, 7))
        segs = []
        for _ in range(nseg):
            lq = int(rng.choice(lqs))
            hist = int(rng.choice([0, 1, 15, 16, 17, 31, 32, 33, 64, 100]))
            segs.append((lq, lq + hist))
        hq = int(rng.choice([1, 2, 3, 4]))
        hkv = hq if hq != 4 or c % 2 else 2
        d = 8 if c % 3 else 64
        dtype = W.F32 if c % 2 else W.BF16
        cases.append((segs, hq, hkv, d, dtype, c))
    cases.append(([(3, 20), (17, 17), (1, 49)], 4, 2, 8, W.F32, 99))  # GQA, group 2
    return cases


def pin_brute_force(orc, quick=False):
    for segs, hq, hkv, d, dtype, seed in brute_cases(quick):
        spec, meta = W.custom_step(segs, hq, hkv, d, dtype, seed=seed)
        hs = W.host_values(spec, meta, seed=seed)
        out, _, _ = run_step(orc, hs)
        ks, vs = logical_kv(hs)
        ref = O.dense_attention(hs.q, ks, vs, meta.cu_seqlens_q)
        err = np.max(np.abs(ref - out))
        assert err <= 1e-12, (segs, hq, hkv, d, dtype, err)


# ------------------------------------------------------------------------ P5
def pin_block_table_fingerprint(orc):
    """K = 0 makes the weights uniform; V channel 0 holds (position mod 256)
    and channel 1 holds (position // 256), both exact in bf16.  Every row is
    then the exact prefix mean of those integer sequences: any wrong page or
    offset shows.  Shuffling physical ids keeps the output bitwise."""
    segs = [(1, 700), (40, 1000), (1, 17), (16, 300)]
    spec, meta = W.custom_step(segs, 2, 2, 8, W.BF16, seed=12)
    hs = W.host_values(spec, meta, seed=12)
    p, hkv = meta.page_size, spec.num_kv_heads
    zero = W.f32_to_bf16_bits(np.zeros(1, np.float32))[0]
    hs.k_cache[:] = zero
    hs.key[:] = zero

    def enc(pos):
        a = np.zeros((len(pos), hkv, spec.head_dim), np.float32)
        a[:, :, 0] = (pos % 256)[:, None]
        a[:, :, 1] = (pos // 256)[:, None]
        return W.f32_to_bf16_bits(a)

    vflat = hs.v_cache.reshape(-1, hkv, spec.head_dim)
    for b, (lq, lk) in enumerate(segs):
        pos = np.arange(lk - lq)
        slots = meta.block_table[b, pos // p].astype(np.int64) * p + pos % p
        vflat[slots] = enc(pos)
        r0 = meta.cu_seqlens_q[b]
        hs.value[r0:r0 + lq] = enc(np.arange(lk - lq, lk))
    out, kc, vc = run_step(orc, hs)
    for b, (lq, lk) in enumerate(segs):
        r0 = meta.cu_seqlens_q[b]
        for i in range(lq):
            n = lk - lq + i + 1
            m0 = Fraction(sum(j % 256 for j in range(n)), n)
            m1 = Fraction(sum(j // 256 for j in range(n)), n)
            assert abs(out[r0 + i, :, 0] - float(m0)).max() < 1e-12, (b, i)
            assert abs(out[r0 + i, :, 1] - float(m1)).max() < 1e-12, (b, i)
    # same logical content under a different physical placement
    perm = np.random.default_rng(1).permutation(meta.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    bt2 = np.where(meta.block_table >= 0, perm[np.maximum(meta.block_table, 0)], -1)
    out2 = orc.attention(hs.q, kc2, vc2, meta.cu_seqlens_q, meta.seqlens_k, bt2)
    assert np.array_equal(out, out2)


# ------------------------------------------------------------------------ P6
def pin_nan_hygiene(orc):
    """NaN in unused tail slots, spare pages and (before the append) new-token
    slots never reaches an output."""
    segs = [(5, 21), (1, 18), (16, 16), (1, 1)]
    spec, meta = W.custom_step(segs, 2, 2, 8, W.BF16, seed=13)
    hs = W.host_values(spec, meta, seed=13, poison=True)
    out, _, _ = run_step(orc, hs)
    assert np.all(np.isfinite(out))
    clean = W.host_values(spec, meta, seed=13, poison=False)
    out2, _, _ = run_step(orc, clean)
    assert np.array_equal(out, out2)


# ------------------------------------------------------------------------ append / slots
def pin_append(orc):
    """The append moves exactly the new rows into their slots, byte for byte;
    every other byte of both pools is unchanged; negative slots are skipped."""
    for dtype in (W.F32, W.BF16):
        segs = [(5, 21), (1, 18), (16, 40)]
        spec, meta = W.custom_step(segs, 3, 3, 8, dtype, seed=14)
        hs = W.host_values(spec, meta, seed=14)
        kc, vc = hs.k_cache.copy(), hs.v_cache.copy()
        sm = meta.slot_mapping.copy()
        sm[3] = -1
        orc.append(hs.key, hs.value, sm, kc, vc)
        ek, ev = hs.k_cache.copy(), hs.v_cache.copy()
        keep = sm >= 0
        ek.reshape(-1, 3, 8)[sm[keep]] = hs.key[keep]
        ev.reshape(-1, 3, 8)[sm[keep]] = hs.value[keep]
        assert kc.tobytes() == ek.tobytes() and vc.tobytes() == ev.tobytes()


def pin_check_slots(orc):
    spec, meta = W.make_step(2)
    args = (meta.cu_seqlens_q, meta.seqlens_k, meta.block_table)
    assert orc.check_slots(*args, meta.slot_mapping, meta.page_size, meta.num_blocks) == 0
    bad = meta.slot_mapping.copy()
    bad[[0, 1]] = bad[[1, 0]]
    assert orc.check_slots(*args, bad, meta.page_size, meta.num_blocks) == 2
    dup = meta.slot_mapping.copy()
    dup[5] = dup[6]
    assert orc.check_slots(*args, dup, meta.page_size, meta.num_blocks) < 0


QUICK_PINS = [pin_worked_example_metadata, pin_worked_example_visibility,
              pin_worked_example_perturbation, pin_textbook_causal, pin_decode_unmasked,
              pin_prefix_means, pin_single_key, pin_constant_values_and_bounds,
              lambda orc: pin_brute_force(orc, quick=True), pin_block_table_fingerprint,
              pin_nan_hygiene, pin_append, pin_check_slots]
