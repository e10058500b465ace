"""HIP path (through the C ABI) against the CPU oracle, element by element.

KV append: bit-exact.  Attention: fp32 max |err| <= 1e-4; bf16 max |err| <=
2e-2 and relative L2 error <= 1e-2.  Inputs are seeded and synthetic with the
shapes of the five workload configs plus a sweep of small ragged shapes; cache
slots no kernel may read (tails of last pages, spare pages, new-token slots
before the append) hold NaN.
"""
import numpy as np
import pytest

from chunked_prefill_mixed_hybrid_amd import binding as B
from chunked_prefill_mixed_hybrid_amd import workload as W
import gpu_support as G
import oracle as O
from oracle import sample as OS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    yield
    import torch
    torch.cuda.empty_cache()


def _free():
    import gc
    import torch
    gc.collect()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- small sweep
SWEEP = [
    # (segments (Lq, Lk), Hq, Hkv, D, dtype, seed)
    ([(1, 1), (1, 17), (1, 300), (1, 64), (1, 65)], 4, 4, 128, W.BF16, 1),
    ([(130, 130)], 2, 2, 128, W.BF16, 2),
    ([(200, 1000)], 2, 2, 128, W.BF16, 3),
    ([(1, 500), (129, 700), (1, 33), (2, 2), (17, 40)], 4, 4, 64, W.BF16, 4),
    ([(1, 500), (129, 700), (1, 33), (2, 2), (17, 40)], 3, 3, 64, W.F32, 5),
    ([(1, 77), (100, 333), (1, 1)], 2, 2, 128, W.F32, 6),
    ([(1, 900), (70, 300), (1, 2)], 8, 2, 128, W.BF16, 7),
    ([(0, 5), (3, 10), (1, 7), (0, 0)], 4, 4, 128, W.BF16, 8),
    ([(1, 5000), (1, 3000), (64, 64)], 4, 4, 128, W.BF16, 9),
    ([(128, 128), (256, 1024), (1, 1024)], 4, 4, 128, W.BF16, 10),
    ([(1, 4097), (33, 4129)], 64, 64, 128, W.BF16, 11),
    ([(5, 5), (1, 2000), (300, 2300)], 2, 1, 64, W.F32, 12),
    # chunk lengths one past a tile multiple, as in the tile-quantisation sweep
    ([(1025, 2561), (1, 3000), (1, 700)], 8, 8, 128, W.BF16, 13),
    ([(1153, 1153), (1, 64)], 4, 4, 128, W.BF16, 14),
    # bf16 decode rows of heads past the last one (6 heads: the second group of
    # 4 has 2), GQA groups of 2 and of 8
    ([(1, 1), (1, 40), (1, 700), (1, 257), (20, 90)], 6, 3, 128, W.BF16, 15),
    ([(1, 3000), (1, 65), (1, 16), (40, 40)], 16, 2, 64, W.BF16, 16),
    # fp32 with as many heads as chunk queue groups (one head per group)
    ([(1, 300), (140, 600), (1, 1), (33, 33)], 8, 8, 64, W.F32, 17),
    # bf16 chunk with more tiles (9 x 64 heads) than the grid has workgroups:
    # the instance whose chunk items claim their successor when done
    ([(1100, 1200), (1, 700), (1, 33)], 64, 64, 128, W.BF16, 18),
]


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_small_sweep(case):
    segs, hq, hkv, d, dt, seed = SWEEP[case]
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=seed)
    hs = W.host_values(spec, meta, seed=seed)
    ds = _dev(hs)
    ref, kc_ref, vc_ref = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    G.note(f"small_sweep case={case} segs={segs} H={hq}/{hkv} D={d} {dt}")
    out = G.gpu_step(ds)
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, dt, f"sweep case {case}")


def _dev(hs):
    return W.to_device(hs, "cuda")


# ---------------------------------------------------------------- random steps
# Seeded random mixed steps through hybrid_step_fwd: 1-40 segments -- decodes
# (history 1..6000), at most 3 chunks (2..700 rows at history 0..3000) and
# empty segments -- 1-8 KV heads in GQA groups of 1, 2 or 4, D 64 or 128, bf16
# or fp32.  Pools bit-exact, the whole output within the oracle's tolerance.
def _random_step(case):
    rng = np.random.default_rng(7000 + case)
    segs, chunks = [], 0
    for _ in range(int(rng.integers(1, 41))):
        u = rng.random()
        if u < 0.3 and chunks < 3:
            chunks += 1
            lq = int(rng.integers(2, 701))
            segs.append((lq, lq + int(rng.integers(0, 3001))))
        elif u < 0.93:
            segs.append((1, int(rng.integers(1, 6001))))
        else:
            segs.append((0, int(rng.integers(0, 41))))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    dt = W.F32 if rng.random() < 0.3 else W.BF16
    return segs, hq, hkv, d, dt


@pytest.mark.parametrize("case", range(40))
def test_random_step(case):
    segs, hq, hkv, d, dt = _random_step(case)
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=7000 + case)
    hs = W.host_values(spec, meta, seed=7000 + case)
    ds = _dev(hs)
    ref, kc_ref, vc_ref = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    G.note(f"random step {case}: {len(segs)} segments, total_q {meta.total_q}, H={hq}/{hkv} D={d} {dt}")
    out = _step(ds, None)
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, dt, f"random step {case}")


def _random_prefill(case):
    """A seeded one-segment bf16 step with at least one (256-row tile, head)
    pair per CU of a 256-CU device, so that it takes the one-segment prefill
    kernel: Lq spread over partial-tile sizes, with or without history."""
    rng = np.random.default_rng(7500 + case)
    hq = int(rng.choice([64, 128]))
    hkv = hq // int(rng.choice([1, 2, 4, 8]))
    lq = int(rng.integers(256 * (256 // hq - 1) + 1, 1400))
    h0 = 0 if rng.random() < 0.4 else int(rng.integers(1, 1500))
    return [(lq, lq + h0)], hq, hkv, int(rng.choice([64, 128]))


@pytest.mark.parametrize("case", range(12))
def test_random_one_segment_prefill(case):
    """Random one-segment prefills through hybrid_step_fwd: the first tile's
    missing rows (256 ceil(Lq / 256) - Lq of them) vary from case to case."""
    segs, hq, hkv, d = _random_prefill(case)
    spec, meta = W.custom_step(segs, hq, hkv, d, W.BF16, seed=7500 + case)
    hs = W.host_values(spec, meta, seed=7500 + case)
    ds = _dev(hs)
    ref, kc_ref, vc_ref = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    lq = segs[0][0]
    G.note(f"random one-segment prefill {case}: segs={segs} H={hq}/{hkv} D={d} "
           f"missing rows {(lq + 255) // 256 * 256 - lq} prefill kernel={_prefill_expected(meta, hq, W.BF16)}")
    out = _step(ds, None)
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, W.BF16, f"random one-segment prefill {case}")


# ---------------------------------------------------------------- chunk KV splits
# Few, long chunk tiles and little decode work: the planner cuts every chunk
# tile into key ranges whose partial results the last range to finish merges.
SPLIT_CASES = [
    # (segments (Lq, Lk), Hq, Hkv, D, dtype, seed)
    ([(200, 1000)], 2, 2, 128, W.BF16, 21),
    ([(1000, 1000)], 1, 1, 64, W.BF16, 22),              # no history: empty late ranges
    ([(130, 8000)], 1, 1, 64, W.BF16, 23),               # many ranges, ragged last tile
    ([(300, 3000), (1, 100)], 2, 2, 128, W.F32, 24),
    ([(1, 700), (257, 2900), (1, 33)], 4, 2, 64, W.F32, 25),   # GQA
    ([(77, 5000), (1, 5), (400, 1400)], 2, 2, 128, W.BF16, 26),
    # fp32, one head: its (tile, range) pairs are dealt over all 8 chunk queues
    ([(300, 6000), (1, 50), (1, 2)], 1, 1, 64, W.F32, 27),
    # fp32, three heads: two sub-groups per head, two of the eight queues empty
    ([(600, 4000), (1, 77), (129, 129)], 3, 3, 64, W.F32, 28),
    # fp32 at D = 128 with GQA: the split instance at the larger head size
    ([(1, 500), (260, 3000), (1, 40)], 4, 2, 128, W.F32, 29),
]


@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
def test_chunk_split(case):
    segs, hq, hkv, d, dt, seed = SPLIT_CASES[case]
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=seed)
    hs = W.host_values(spec, meta, seed=seed)
    ds = _dev(hs)
    ref, kc_ref, vc_ref = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    G.note(f"chunk_split case={case} segs={segs} H={hq}/{hkv} D={d} {dt}")
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, hq, d)
    out = G.gpu_step(ds, workspace=ws)
    hdr = G.plan_header(ws)
    assert hdr["chunk_split"] > 1, hdr
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, dt, f"split case {case}")
    # a second call on the same workspace (counters left over from the first)
    out2 = G.gpu_step(ds, workspace=ws, append=False)
    G.compare(G.to_f64(out2), ref, dt, f"split case {case}, second call")


# ---------------------------------------------------------------- one-segment prefill kernel
# A bf16 step that is one prefill chunk, with at least one (256-row tile, head)
# pair per CU, runs a kernel of its own (64 query rows per wave, one workgroup
# per CU): no planner, no combine, and the workspace is left untouched, which
# is how the tests see which path ran.  Ragged last tiles, histories off the
# page and key-step grid, GQA, D = 64 and 128.
PREFILL_CASES = [
    # (segments (Lq, Lk), Hq, Hkv, D, dtype, seed)
    ([(1000, 1000)], 64, 64, 128, W.BF16, 41),
    ([(777, 3000)], 64, 8, 128, W.BF16, 42),      # GQA 8, history 2223
    ([(300, 300)], 128, 128, 64, W.BF16, 43),
    ([(513, 530)], 128, 128, 128, W.BF16, 44),    # one row in the last tile, history 17
    ([(1000, 1000)], 32, 32, 128, W.BF16, 45),    # 4 x 32 pairs: below one per CU, fused path
    ([(1024, 1500)], 64, 16, 128, W.BF16, 46),    # whole tiles only, GQA 4
    ([(200, 700)], 256, 32, 64, W.BF16, 47),      # one partial tile per head, GQA 8
]
_SENTINEL = 0x5A


def _prefill_expected(meta, hq, dt):
    """Whether the step takes the one-segment prefill kernel on this device."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-int(meta.max_seqlen_q) // 256)
    return dt == W.BF16 and meta.num_seqs == 1 and meta.max_seqlen_q > 1 and tiles * hq >= cus


def _marked_workspace(meta, hq, d):
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, hq, d)
    ws.fill_(_SENTINEL)
    return ws


def _workspace_untouched(ws):
    return bool((ws[:256] == _SENTINEL).all().item())


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_one_segment_prefill(case):
    import torch
    segs, hq, hkv, d, dt, seed = PREFILL_CASES[case]
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=seed)
    hs = W.host_values(spec, meta, seed=seed)
    ds = _dev(hs)
    ref, kc_ref, vc_ref = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    wide = _prefill_expected(meta, hq, dt)
    G.note(f"one-segment prefill case={case} segs={segs} H={hq}/{hkv} D={d} prefill kernel={wide}")
    ws = _marked_workspace(meta, hq, d)
    out = G.gpu_step(ds, workspace=ws)
    assert _workspace_untouched(ws) == wide
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, dt, f"prefill case {case}")
    # the same step through hybrid_step_fwd (append inside) and through the
    # packed-K/V entry point: byte-identical
    ds_b = _dev(hs)
    ws_b = _marked_workspace(meta, hq, d)
    out_b = _step(ds_b, ws_b)
    assert _workspace_untouched(ws_b) == wide
    assert torch.equal(out_b.view(torch.uint8), out.view(torch.uint8))
    kc_b, vc_b = G.host_pools(ds_b)
    assert kc_b.tobytes() == kc.tobytes() and vc_b.tobytes() == vc.tobytes()
    k, v, cu_k = G.contiguous_kv(ds)
    out_c = B.varlen_attn_fwd(ds.q, k, v, ds.cu_seqlens_q, cu_k, meta.max_seqlen_q, meta.max_seqlen_k)
    torch.cuda.synchronize()
    assert torch.equal(out_c.view(torch.uint8), out.view(torch.uint8))


@pytest.mark.parametrize("case", [1, 3, 4])
def test_one_segment_prefill_packed_keys_at_an_offset(case):
    """varlen_attn_fwd on one segment whose keys start past row 0 of the packed
    buffers (NaN rows before and after them): byte-identical to the paged call."""
    import torch
    segs, hq, hkv, d, dt, seed = PREFILL_CASES[case]
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=seed)
    ds = _dev(W.host_values(spec, meta, seed=seed))
    G.note(f"one-segment prefill, packed keys at row 37: case={case} segs={segs}")
    paged = G.gpu_step(ds)
    k, v, cu_k = G.contiguous_kv(ds)
    lead = torch.full((37,) + tuple(k.shape[1:]), float("nan"), dtype=k.dtype, device=k.device)
    k2, v2 = torch.cat([lead, k]).contiguous(), torch.cat([lead, v]).contiguous()
    ws = _marked_workspace(meta, hq, d)
    out = B.varlen_attn_fwd(ds.q, k2, v2, ds.cu_seqlens_q, cu_k + 37, meta.max_seqlen_q,
                            meta.max_seqlen_k, workspace=ws)
    torch.cuda.synchronize()
    assert _workspace_untouched(ws) == _prefill_expected(meta, hq, dt)
    assert torch.equal(out.view(torch.uint8), paged.view(torch.uint8))


def test_one_segment_prefill_appends_tokens_outside_the_segment():
    """hybrid_step_fwd on a one-segment step whose token list also holds rows
    past the segment (a padding token, and tokens bound for unused slots):
    every token with a valid slot is appended, as paged_kv_append does, and
    the segment's output is unchanged."""
    import torch
    spec, meta = W.custom_step([(1000, 1000)], 64, 64, 128, W.BF16, seed=47)
    hs = W.host_values(spec, meta, seed=47)
    ds = _dev(hs)
    extra = 6
    rng = np.random.default_rng(47)
    free = np.setdiff1d(meta.poison_slots, meta.slot_mapping)  # slots no segment owns or appends to
    slots = np.concatenate([meta.slot_mapping, [-1], rng.choice(free, extra - 1, replace=False)])
    g = torch.Generator(device="cuda")
    g.manual_seed(48)
    pad = lambda x: torch.cat([x, torch.randn((extra,) + tuple(x.shape[1:]), generator=g, device="cuda").to(x.dtype)])
    ds2 = W.DeviceStep(spec, meta, pad(ds.q), pad(ds.key), pad(ds.value), ds.k_cache.clone(), ds.v_cache.clone(),
                       ds.cu_seqlens_q, ds.seqlens_k, ds.block_table,
                       torch.from_numpy(slots.astype(np.int32)).cuda())
    G.note("one-segment prefill: 6 tokens past the segment")
    ref_k, ref_v = ds.k_cache.clone(), ds.v_cache.clone()
    B.paged_kv_append(ds2.key, ds2.value, ds2.slot_mapping, ref_k, ref_v)
    out = torch.empty_like(ds2.q)
    B.hybrid_step_fwd(ds2.key, ds2.value, ds2.slot_mapping, ds2.q, ds2.k_cache, ds2.v_cache,
                      ds2.cu_seqlens_q, ds2.seqlens_k, ds2.block_table, meta.max_seqlen_q,
                      meta.max_seqlen_k, out=out)
    torch.cuda.synchronize()
    assert torch.equal(ds2.k_cache.view(torch.int16), ref_k.view(torch.int16))
    assert torch.equal(ds2.v_cache.view(torch.int16), ref_v.view(torch.int16))
    ref_out = G.gpu_step(ds)
    assert torch.equal(out[:1000].view(torch.uint8), ref_out.view(torch.uint8))


def test_one_segment_prefill_declared_max_above_rows():
    """max_seqlen_q is an upper bound (at most max_seqlen_k): tiles past the
    segment's rows do nothing."""
    import torch
    spec, meta = W.custom_step([(700, 1500)], 64, 64, 128, W.BF16, seed=46)
    hs = W.host_values(spec, meta, seed=46)
    ds = _dev(hs)
    ref, _, _ = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    G.note("one-segment prefill: 700 rows, max_seqlen_q 1280")
    B.paged_kv_append(ds.key, ds.value, ds.slot_mapping, ds.k_cache, ds.v_cache)
    ws = _marked_workspace(meta, 64, 128)
    out = torch.full_like(ds.q, float("nan"))
    B.hybrid_attn_fwd(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q, ds.seqlens_k, ds.block_table,
                      1280, meta.max_seqlen_k, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert _workspace_untouched(ws) == _prefill_expected(W.StepMeta(
        meta.cu_seqlens_q, meta.seqlens_k, meta.block_table, None, meta.num_blocks,
        meta.page_size, 1280, meta.max_seqlen_k), 64, W.BF16)
    G.compare(G.to_f64(out), ref, W.BF16, "prefill, declared max above the rows")


# ---------------------------------------------------------------- two-launch baseline
# The chunk role and the decode role in separate launches (back to back, or on
# two streams): the same plan and items as the fused launch, so the output is
# bitwise the fused one.
TWO_LAUNCH_CASES = [("sweep", 3), ("sweep", 6), ("sweep", 9), ("sweep", 11), ("split", 3),
                    ("split", 5),
                    ("sweep", 17),  # bf16 instance with deferred chunk claims
                    ("split", 6)]   # fp32, one head: queue sub-groups, equal key ranges


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("case", range(len(TWO_LAUNCH_CASES)))
def test_two_launch_matches_fused(case, two_streams):
    import torch
    kind, idx = TWO_LAUNCH_CASES[case]
    segs, hq, hkv, d, dt, seed = (SWEEP if kind == "sweep" else SPLIT_CASES)[idx]
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=seed)
    hs = W.host_values(spec, meta, seed=seed)
    ds = _dev(hs)
    ref, _, _ = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    G.note(f"two_launch {kind} case={idx} two_streams={two_streams} segs={segs}")
    fused = G.gpu_step(ds)
    two = B.hybrid_attn_fwd_two_launch(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q, ds.seqlens_k,
                                       ds.block_table, meta.max_seqlen_q, meta.max_seqlen_k,
                                       two_streams=two_streams)
    torch.cuda.synchronize()
    assert torch.equal(two.view(torch.uint8), fused.view(torch.uint8))  # byte for byte
    G.compare(G.to_f64(two), ref, dt, f"two-launch {kind} {idx}")


def test_two_launch_config2_matches_fused():
    import torch
    spec, meta = W.make_step(2)
    ds = W.device_values(spec, meta, seed=0)
    G.note("two_launch config2 serial and two streams")
    fused = G.gpu_step(ds)
    for two_streams in (False, True):
        two = B.hybrid_attn_fwd_two_launch(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q,
                                           ds.seqlens_k, ds.block_table, meta.max_seqlen_q,
                                           meta.max_seqlen_k, two_streams=two_streams)
        torch.cuda.synchronize()
        assert torch.equal(two.view(torch.int16), fused.view(torch.int16)), two_streams
    del ds
    _free()


# ---------------------------------------------------------------- contiguous K/V
# varlen_attn_fwd over each segment's keys packed into one buffer (segments
# start at arbitrary rows, NaN rows follow the last one): the same plan and
# arithmetic as the paged call (chunk splits included), so the output is
# byte-identical to it.
CONTIG_CASES = [("sweep", 0), ("sweep", 3), ("sweep", 4), ("sweep", 6), ("sweep", 7),
                ("sweep", 9), ("sweep", 10), ("sweep", 11), ("sweep", 12), ("sweep", 13),
                ("sweep", 14), ("sweep", 15), ("split", 1),
                ("sweep", 17), ("split", 3), ("split", 6)]


@pytest.mark.parametrize("case", range(len(CONTIG_CASES)))
def test_contiguous_kv_matches_paged(case):
    import torch
    kind, idx = CONTIG_CASES[case]
    segs, hq, hkv, d, dt, seed = (SWEEP if kind == "sweep" else SPLIT_CASES)[idx]
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=seed)
    hs = W.host_values(spec, meta, seed=seed)
    ds = _dev(hs)
    ref, _, _ = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    G.note(f"contiguous kv {kind} case={idx} segs={segs}")
    paged = G.gpu_step(ds)  # appends, so the pools hold every key
    k, v, cu_k = G.contiguous_kv(ds)
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, hq, d)
    out = B.varlen_attn_fwd(ds.q, k, v, ds.cu_seqlens_q, cu_k, meta.max_seqlen_q, meta.max_seqlen_k,
                            workspace=ws)
    torch.cuda.synchronize()
    G.compare(G.to_f64(out), ref, dt, f"contiguous {kind} {idx}")
    assert torch.equal(out.view(torch.uint8), paged.view(torch.uint8))
    if kind == "split":
        assert G.plan_header(ws)["chunk_split"] > 1  # splits work on packed keys too


def test_contiguous_kv_config2():
    import torch
    spec, meta = W.make_step(2)
    ds = W.device_values(spec, meta, seed=0)
    G.note("contiguous kv config2")
    paged = G.gpu_step(ds)
    k, v, cu_k = G.contiguous_kv(ds)
    out = B.varlen_attn_fwd(ds.q, k, v, ds.cu_seqlens_q, cu_k, meta.max_seqlen_q, meta.max_seqlen_k)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), paged.view(torch.uint8))
    del ds, k, v
    _free()


# ---------------------------------------------------------------- whole-step entry point
# hybrid_step_fwd = paged_kv_append then hybrid_attn_fwd; the append and the
# small planner share a launch for wide rows (Hkv*D*e >= 2 KB) and <= 64
# segments, the calls run one after the other otherwise.  Pools and output
# must be byte-identical to the two calls, and the output within the oracle's
# tolerance.
STEP_CASES = [("sweep", 10), ("sweep", 12), ("sweep", 0), ("sweep", 4), ("many", 0)]


def _step_case(kind, idx):
    if kind == "sweep":
        return SWEEP[idx]
    # more than one wave of segments: the block-wide planner, separate launches
    segs = [(1, 17 + 37 * i) for i in range(70)] + [(130, 400)]
    return segs, 8, 8, 128, W.BF16, 31


def _step(ds, ws):
    import torch
    m = ds.meta
    out = torch.empty_like(ds.q)
    B.hybrid_step_fwd(ds.key, ds.value, ds.slot_mapping, ds.q, ds.k_cache, ds.v_cache,
                      ds.cu_seqlens_q, ds.seqlens_k, ds.block_table, m.max_seqlen_q,
                      m.max_seqlen_k, out=out, workspace=ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", STEP_CASES)
def test_step_entry_matches_two_calls(case):
    import torch
    segs, hq, hkv, d, dt, seed = _step_case(*case)
    spec, meta = W.custom_step(segs, hq, hkv, d, dt, seed=seed)
    hs = W.host_values(spec, meta, seed=seed)
    G.note(f"step entry case={case} segs={len(segs)} H={hq}/{hkv} D={d} {dt}")
    ds_a, ds_b = _dev(hs), _dev(hs)
    ref, kc_ref, vc_ref = G.oracle_full(ds_a, hs.k_cache, hs.v_cache)
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, hq, d)
    out_a = G.gpu_step(ds_a, workspace=ws)
    out_b = _step(ds_b, ws)
    assert (out_b.view(torch.uint8).cpu().numpy().tobytes() ==
            out_a.view(torch.uint8).cpu().numpy().tobytes())
    kc, vc = G.host_pools(ds_b)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out_b), ref, dt, f"step entry {case}")


def test_step_entry_config2():
    spec, meta = W.make_step(2)
    ds = W.device_values(spec, meta, seed=0)
    kc0, vc0 = G.host_pools(ds)
    ref, kc_ref, vc_ref = G.oracle_full(ds, kc0, vc0)
    del kc0, vc0
    G.note("step entry config2 bf16 H=32 D=128 (append and planner in one launch)")
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, spec.num_heads,
                           spec.head_dim)
    out = _step(ds, ws)
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, W.BF16, "step entry config 2")
    del ds
    _free()


# ---------------------------------------------------------------- full configs
def test_config1_worked_example():
    spec, meta = W.make_step(1)
    hs = W.host_values(spec, meta, seed=0)
    ds = _dev(hs)
    ref, kc_ref, vc_ref = G.oracle_full(ds, hs.k_cache, hs.v_cache)
    G.note("config1 worked example fp32 H=2 D=64")
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, spec.num_heads,
                           spec.head_dim)
    out = G.gpu_step(ds, workspace=ws)
    assert G.plan_header(ws)["chunk_split"] > 1  # 30 long tiles on a whole GPU: split
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, W.F32, "config 1")


def test_config2_full():
    spec, meta = W.make_step(2)
    ds = W.device_values(spec, meta, seed=0)
    kc0, vc0 = G.host_pools(ds)
    ref, kc_ref, vc_ref = G.oracle_full(ds, kc0, vc0)
    del kc0, vc0
    G.note("config2 2x512 chunks + 30 decodes bf16 H=32 D=128")
    out = G.gpu_step(ds)
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, W.BF16, "config 2")
    del ds
    _free()


def _equal_in_slabs(x, y, slab=1 << 29) -> bool:
    """Bitwise equality of two big device tensors, compared in slabs (no
    temporary the size of the pools)."""
    import torch
    fx, fy = x.view(-1).view(torch.int16), y.view(-1).view(torch.int16)
    if fx.numel() != fy.numel():
        return False
    for s0 in range(0, fx.numel(), slab):
        if not torch.equal(fx[s0:s0 + slab], fy[s0:s0 + slab]):
            return False
    return True


def _edge_rows(n, rng, extra=6):
    """The first and last row of every 128-row query tile, the middle row and
    `extra` random rows of a chunk of n rows."""
    base = {0, 1, n - 1, n // 2}
    for t in range(128, n, 128):
        base |= {t - 1, t}
    base = {r for r in base if 0 <= r < n}
    base |= set(rng.choice(n, size=min(extra, n), replace=False).tolist())
    return sorted(base)


def _config_parity(config, extra_chunk_rows, batch_bytes=4 << 30, require_tail=False):
    """Whole-pool append check plus oracle parity of EVERY decode row (all
    heads) and of the first and last row of every chunk tile (plus random
    rows) of a big workload step.  Pages reach the host a few segments at a
    time, from device copies of the pools taken before the append."""
    import torch
    spec, meta = W.make_step(config)
    ds = W.device_values(spec, meta, seed=0)
    lq = np.diff(meta.cu_seqlens_q)
    rng = np.random.default_rng(100 + config)
    hkv, d = spec.num_kv_heads, spec.head_dim
    k_before, v_before = ds.k_cache.clone(), ds.v_cache.clone()
    G.note(f"config{config}: GPU step ({meta.num_seqs} segments, {meta.total_q} rows)")
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, spec.num_heads, d)
    out = G.gpu_step(ds, workspace=ws)
    hdr = _check_plan_arrays(ws, meta, spec.num_heads)
    G.note(f"config{config}: decode split {hdr['split']}, {hdr['n_dec_full']} full-split items, "
           f"{hdr['n_dec_items'] - hdr['n_dec_full']} tail-piece items")
    if require_tail:
        assert hdr["n_dec_items"] > hdr["n_dec_full"], hdr
    sel_rows = np.zeros(meta.total_q, np.uint8)
    for b in range(meta.num_seqs):
        r0, n = int(meta.cu_seqlens_q[b]), int(lq[b])
        if n == 1:
            sel_rows[r0] = 1
        elif n > 1:
            sel_rows[r0 + np.array(_edge_rows(n, rng, extra_chunk_rows))] = 1
    # chunk segments first (the longest rows), then the decodes in batches
    order = [b for b in range(meta.num_seqs) if lq[b] > 1] + \
            [b for b in range(meta.num_seqs) if lq[b] == 1]
    batches = OS.segment_batches(meta, order, batch_bytes, hkv * d * 2)
    err_sq = ref_sq = 0.0
    max_abs = 0.0
    checked = 0
    for i, segs in enumerate(batches):
        smp = OS.SampledStep(meta, ds.q, ds.key, ds.value, k_before, v_before, segs)
        sel = sel_rows[smp.rows]
        G.note(f"config{config}: oracle batch {i + 1}/{len(batches)}: {len(segs)} segments, "
               f"{int(sel.sum())} rows, {smp.nbytes / 1e9:.2f} GB of pages")
        ref, kc_ref, vc_ref = smp.oracle(row_select=sel)
        # the append of these segments, bit-exact against the oracle's
        kc_got = W.to_host_array(ds.k_cache.index_select(0, smp.page_idx))
        vc_got = W.to_host_array(ds.v_cache.index_select(0, smp.page_idx))
        assert kc_got.tobytes() == kc_ref.tobytes() and vc_got.tobytes() == vc_ref.tobytes(), segs
        del kc_got, vc_got, kc_ref, vc_ref
        got = G.to_f64(out.index_select(0, torch.from_numpy(smp.rows).to(out.device)))
        rows = sel.astype(bool)
        st = G.compare(got[rows], ref[rows], W.BF16, f"config {config} batch {i}")
        max_abs = max(max_abs, st["max_abs"])
        err_sq += float(np.sum((got[rows] - ref[rows]) ** 2))
        ref_sq += float(np.sum(ref[rows] ** 2))
        checked += int(rows.sum())
        del smp, ref, got
    assert checked == int(sel_rows.sum())
    rel = (err_sq / ref_sq) ** 0.5
    G.note(f"config{config}: {checked} rows x {spec.num_heads} heads against the oracle: "
           f"max abs {max_abs:.3e}, rel L2 {rel:.3e}")
    assert max_abs <= G.TOL_BF16_ABS and rel <= G.TOL_BF16_REL
    # every pool slot other than this step's new-token slots is bitwise unchanged
    slots = ds.slot_mapping.long()
    for before, after, new in ((k_before, ds.k_cache, ds.key), (v_before, ds.v_cache, ds.value)):
        a16 = after.view(-1, hkv * d).view(torch.int16)
        assert torch.equal(a16.index_select(0, slots), new.reshape(-1, hkv * d).view(torch.int16))
        before.view(-1, hkv * d).index_copy_(0, slots, new.reshape(-1, hkv * d))
        assert _equal_in_slabs(before, after)
    del k_before, v_before, ds, out
    _free()
    return {"max_abs": max_abs, "rel_norm": rel, "rows": checked}


@pytest.mark.timeout(900)
def test_config3_decode_heavy():
    _config_parity(3, 6)


@pytest.mark.timeout(900)
def test_config4_long_context():
    _config_parity(4, 4, require_tail=True)  # long decodes: the queue ends with tail pieces


@pytest.mark.timeout(900)
def test_config5_budget2048():
    _config_parity(5, 12)


# ---------------------------------------------------------------- more segments than the LDS holds
def test_many_segments_budget_step():
    """A budget-2048 step of 2040 decodes and one 8-token chunk: 2041 segments
    take the block-wide planner's multi-pass prefix loop (more than 1024) and
    the attention kernel's global item lookup (more than 512).  Whole output
    against the oracle, append bit-exact over the whole pool, and the
    planner's prefix arrays against their definitions."""
    import torch
    rng = np.random.default_rng(41)
    segs = [(1, int(h) + 1) for h in rng.integers(0, 300, 2040, endpoint=True)] + [(8, 130)]
    hq, d = 8, 128
    spec, meta = W.custom_step(segs, hq, hq, d, W.BF16, seed=41)
    ds = W.device_values(spec, meta, seed=41)
    kc0, vc0 = G.host_pools(ds)
    ref, kc_ref, vc_ref = G.oracle_full(ds, kc0, vc0)
    del kc0, vc0
    G.note(f"many segments: {meta.num_seqs} segments, H={hq} D={d} bf16")
    ws = B.alloc_workspace(meta.num_seqs, meta.total_q, meta.max_seqlen_k, hq, d)
    out = G.gpu_step(ds, workspace=ws)
    kc, vc = G.host_pools(ds)
    assert kc.tobytes() == kc_ref.tobytes() and vc.tobytes() == vc_ref.tobytes()
    G.compare(G.to_f64(out), ref, W.BF16, "many segments")
    _check_plan_arrays(ws, meta, hq)
    del ds
    _free()


def _check_plan_arrays(ws, meta, hq):
    """The planner's per-segment arrays in the workspace (after the 256-byte
    header: chunk (tile, range) pairs per head, decode full-split items,
    partial slots, key lengths, decode tail-piece items) against their
    definitions: a decode segment of Lk keys at split S has ceil(Lk / S) full
    splits, or, when S >= 2048, ceil(Lk / S) - 1 full splits and the rest in
    pieces of S / 4 keys; each split or piece is one item per group of 4
    heads; partial slots are needed when a segment has more than one."""
    hdr = G.plan_header(ws)
    nseg = meta.num_seqs
    arr = (4 * (nseg + 1) + 255) // 256 * 256
    raw = ws[256:256 + 5 * arr].cpu().numpy().view(np.int32)
    tile_p, dec_p, part_p, _, tail_p = (raw[k * arr // 4:k * arr // 4 + nseg + 1] for k in range(5))
    lqs = np.diff(meta.cu_seqlens_q).astype(np.int64)
    lks = meta.seqlens_k.astype(np.int64)
    split, cs = hdr["split"], hdr["chunk_split"]
    head_groups = (hq + 3) // 4
    n = np.where(lqs == 1, (lks + split - 1) // split, 0)
    if split >= 2048:
        full = np.maximum(n - 1, 0)
        piece = split // 4
        tail = np.where(lqs == 1, (lks - full * split + piece - 1) // piece, 0)
    else:
        full, tail = n, np.zeros_like(n)
    want = [np.where(lqs >= 2, (lqs + 127) // 128 * cs, 0), full * head_groups,
            np.where(full + tail > 1, full + tail, 0), tail * head_groups]
    for got_p, w_p, name in zip((tile_p, dec_p, part_p, tail_p), want,
                                ("tile", "decode", "partial", "tail")):
        ex = np.concatenate([[0], np.cumsum(w_p)])
        assert np.array_equal(got_p.astype(np.int64), ex), (name, split)
    assert hdr["n_dec_full"] == int(dec_p[-1]) and hdr["bad_segments"] == 0
    assert hdr["n_dec_items"] == int(dec_p[-1]) + int(tail_p[-1])
    return hdr


# ---------------------------------------------------------------- chunk invariance
def test_chunk_invariance_10000_prompt():
    """The 10000-token prompt prefilled as 4 x 2048 + 1808 gives the same KV
    bytes as one full prefill and outputs within tolerance of it and of the
    oracle (H=64, D=128, bf16, as in the budget-2048 workload)."""
    import torch
    steps = W.chunked_prompt_steps(10000, 2048)
    spec, meta = W.custom_step([(10000, 10000)], 64, 64, 128, W.BF16, seed=21)
    full = W.device_values(spec, meta, seed=21)
    k0, v0 = full.k_cache.clone(), full.v_cache.clone()
    kc_host, vc_host = G.host_pools(full)
    G.note("chunk invariance: full 10000-token prefill")
    out_full = G.gpu_step(full)
    outs = []
    for lq, lk in steps:
        h0 = lk - lq
        ds = W.DeviceStep(spec, meta, full.q[h0:lk], full.key[h0:lk], full.value[h0:lk], k0, v0,
                          torch.tensor([0, lq], dtype=torch.int32, device="cuda"),
                          torch.tensor([lk], dtype=torch.int32, device="cuda"),
                          full.block_table, full.slot_mapping[h0:lk].contiguous())
        ds.meta = W.StepMeta(np.array([0, lq], np.int32), np.array([lk], np.int32),
                             meta.block_table, meta.slot_mapping[h0:lk], meta.num_blocks,
                             meta.page_size, lq, lk)
        G.note(f"chunk invariance: step Lq={lq} Lk={lk}")
        outs.append(G.gpu_step(ds))
    out_chunked = torch.cat(outs)
    assert torch.equal(k0.view(torch.int16), full.k_cache.view(torch.int16))
    assert torch.equal(v0.view(torch.int16), full.v_cache.view(torch.int16))
    a, b = G.to_f64(out_chunked), G.to_f64(out_full)
    G.compare(a, b, W.BF16, "chunked vs full")
    rng = np.random.default_rng(5)
    rows = sorted({0, 2047, 2048, 8191, 8192, 9999} | set(rng.choice(10000, 26, replace=False).tolist()))
    sel = np.zeros(10000, np.uint8)
    sel[rows] = 1
    ref, _, _ = G.oracle_full(full, kc_host, vc_host, row_select=sel)
    G.compare(a[rows], ref[rows], W.BF16, "chunked vs oracle")
    G.compare(b[rows], ref[rows], W.BF16, "full vs oracle")
    G.note(f"chunk invariance: chunked == full bitwise: {bool(np.array_equal(a, b))}")


# ---------------------------------------------------------------- properties
def test_repeat_is_deterministic():
    spec, meta = W.make_step(2)
    ds = W.device_values(spec, meta, seed=0)
    G.note("determinism: config 2 twice")
    a = G.gpu_step(ds)
    b = G.gpu_step(ds)
    import torch
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_segment_order_does_not_matter():
    """Each segment sees only its own pages: packing the same segments in
    another order gives bitwise the same rows."""
    import torch
    segs = [(1, 700), (90, 400), (1, 40), (1, 2500), (33, 33)]
    spec, meta = W.custom_step(segs, 4, 4, 128, W.BF16, seed=31)
    hs = W.host_values(spec, meta, seed=31, poison=False)
    ds = _dev(hs)
    G.note("segment order: original")
    out = W.to_host_array(G.gpu_step(ds, append=False))
    order = [3, 0, 4, 2, 1]
    lq = np.diff(meta.cu_seqlens_q)
    rows = np.concatenate([np.arange(meta.cu_seqlens_q[b], meta.cu_seqlens_q[b + 1]) for b in order])
    cu = np.concatenate([[0], np.cumsum(lq[order])]).astype(np.int32)
    ds2 = W.DeviceStep(spec, meta, ds.q[torch.from_numpy(rows).cuda()].contiguous(), None, None,
                       ds.k_cache, ds.v_cache, torch.from_numpy(cu).cuda(),
                       ds.seqlens_k[order].contiguous(), ds.block_table[order].contiguous(), None)
    ds2.meta = W.StepMeta(cu, meta.seqlens_k[order], meta.block_table[order], None,
                          meta.num_blocks, meta.page_size, meta.max_seqlen_q, meta.max_seqlen_k)
    G.note("segment order: permuted")
    out2 = W.to_host_array(G.gpu_step(ds2, append=False))
    assert np.array_equal(out2, out[rows])


def test_workspace_too_small_is_reported():
    import torch
    spec, meta = W.custom_step([(1, 100)], 2, 2, 64, W.F32, seed=1)
    ds = _dev(W.host_values(spec, meta))
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.HybridAttnError) as e:
        B.hybrid_attn_fwd(ds.q, ds.k_cache, ds.v_cache, ds.cu_seqlens_q, ds.seqlens_k,
                          ds.block_table, 1, 100, workspace=ws)
    assert e.value.status == B.HA_ERR_WORKSPACE_TOO_SMALL
