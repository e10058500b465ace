"""Host tests of the token-budget step generator (include/ha_scheduler.h).

Policy from the wangyu.me chunked-prefill page (section on the vLLM
implementation): a per-step token budget, running requests first in admission
order, then the waiting queue; chunk = min(remaining, threshold, budget left).
The page's own numbers are the golden cases: a 10000-token prompt under a 2048
budget runs as 4 x 2048 + 1808, and three decodes riding along a prompt under
a 1024 budget leave 1021 tokens for its chunk.  Then invariants over random
traces, and the oracle on the scheduled steps against the oracle on each
request in one piece (chunk invariance across requests, exact in fp64).
"""
import numpy as np
import pytest

from chunked_prefill_mixed_hybrid_amd import binding as B

PAGE = 16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not B.LIB_PATH.exists():
        from chunked_prefill_mixed_hybrid_amd import build
        build.build()


def sched(budget, blocks=4096, mb=1024, threshold=0, max_seqs=256):
    from chunked_prefill_mixed_hybrid_amd.scheduler import StepScheduler
    return StepScheduler(budget, blocks, mb, long_prefill_token_threshold=threshold,
                         max_seqs=max_seqs)


def run_all(s, limit=100000):
    steps = []
    for _ in range(limit):
        st = s.next_step()
        if st is None:
            return steps
        steps.append(st)
        s.complete()
    raise AssertionError("trace did not finish")


def lq(st):
    return np.diff(st.cu_seqlens_q).tolist()


def test_page_example_10000_prompt_under_2048_budget():
    s = sched(2048)
    s.add(7, 10000, 3)
    steps = run_all(s)
    assert [lq(st) for st in steps] == [[2048], [2048], [2048], [2048], [1808], [1], [1]]
    assert [int(st.seqlens_k[0]) for st in steps] == [2048, 4096, 6144, 8192, 10000, 10001, 10002]
    assert [int(st.first_pos[0]) for st in steps] == [0, 2048, 4096, 6144, 8192, 10000, 10001]
    assert [st.num_sampling for st in steps] == [0, 0, 0, 0, 1, 1, 1]
    assert [st.num_decodes for st in steps] == [0, 0, 0, 0, 0, 1, 1]
    assert s.unfinished == 0 and s.free_blocks == 4096


def test_page_example_three_decodes_and_a_1021_chunk():
    s = sched(1024)
    for r in range(3):
        s.add(r, 10, 5)
    first = s.next_step()
    assert lq(first) == [10, 10, 10]
    s.complete()  # all three sample: they are decoding now
    s.add(3, 5000, 1)
    st = s.next_step()
    assert lq(st) == [1, 1, 1, 1021] and st.total_q == 1024 and st.num_decodes == 3
    assert st.request_ids.tolist() == [0, 1, 2, 3]


def test_running_requests_come_before_the_waiting_queue():
    s = sched(2048)
    s.add(0, 3000, 2)
    s.add(1, 500, 2)
    st = s.next_step()
    assert lq(st) == [2048] and st.request_ids.tolist() == [0]
    s.complete()
    st = s.next_step()  # request 0 finishes its prompt first, request 1 fills the rest
    assert lq(st) == [952, 500] and st.request_ids.tolist() == [0, 1]
    s.complete()
    st = s.next_step()
    assert lq(st) == [1, 1] and st.num_decodes == 2


def test_long_prefill_threshold_bounds_every_chunk():
    s = sched(4096, threshold=1024)
    s.add(0, 3000, 1)
    s.add(1, 1500, 1)
    steps = run_all(s)
    assert [lq(st) for st in steps] == [[1024, 1024], [1024, 476], [952]]


def _check_step(st, budget, pages_of, prev_computed):
    n = np.diff(st.cu_seqlens_q)
    assert st.total_q <= budget and np.all(n >= 1)
    assert np.all(st.seqlens_k == st.first_pos + n)
    assert st.max_seqlen_q == n.max() and st.max_seqlen_k == st.seqlens_k.max()
    t = 0
    used = set()
    for b, rid in enumerate(st.request_ids.tolist()):
        assert rid not in used
        used.add(rid)
        assert prev_computed.get(rid, 0) == st.first_pos[b]  # positions continue where they stopped
        npages = -(-int(st.seqlens_k[b]) // PAGE)
        row = st.block_table[b]
        assert np.all(row[:npages] >= 0) and np.all(row[npages:] == -1)
        pages_of[rid] = row[:npages].tolist()
        for i in range(n[b]):
            pos = st.first_pos[b] + i
            assert st.slot_mapping[t + i] == row[pos // PAGE] * PAGE + pos % PAGE
        t += n[b]
        prev_computed[rid] = int(st.seqlens_k[b])
    live = [p for r in pages_of.values() for p in r]
    assert len(live) == len(set(live))  # no page belongs to two live requests


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_keep_every_invariant(seed):
    rng = np.random.default_rng(seed)
    budget = int(rng.choice([64, 256, 1000, 2048]))
    threshold = int(rng.choice([0, 0, 100, 700]))
    blocks = 2048
    s = sched(budget, blocks=blocks, mb=512, threshold=threshold)
    reqs = {}
    for rid in range(int(rng.integers(1, 25))):
        p, g = int(rng.integers(1, 3000)), int(rng.integers(1, 20))
        reqs[rid] = (p, g)
        s.add(rid, p, g)
    pages_of, computed, finished = {}, {}, []
    late = iter(range(100, 110))
    for step_no in range(100000):
        st = s.next_step()
        if st is None:
            break
        _check_step(st, budget, pages_of, computed)
        # running first: a request admitted this step comes after all running ones
        new = [computed_before == 0 for computed_before in st.first_pos]
        if any(new):
            assert not any(not x for x in new[new.index(True):])
        for rid in s.complete():
            p, g = reqs[rid]
            assert computed[rid] == p + g - 1  # every known token went through once
            finished.append(rid)
            pages_of.pop(rid)
        if step_no % 7 == 3:  # requests keep arriving
            rid = next(late, None)
            if rid is not None:
                p, g = int(rng.integers(1, 500)), int(rng.integers(1, 5))
                reqs[rid] = (p, g)
                s.add(rid, p, g)
    assert sorted(finished) == sorted(reqs) and s.unfinished == 0 and s.free_blocks == blocks


def test_small_pool_shrinks_chunks_and_reports_a_stall():
    s = sched(1024, blocks=10, mb=64)  # 160 tokens of cache
    s.add(0, 100, 2)
    s.add(1, 100, 2)
    st = s.next_step()
    assert lq(st) == [100, 48]  # request 0 holds 7 pages; request 1 fits the 3 left
    s.complete()
    st = s.next_step()  # request 0 decodes into its last page; request 1 has no room
    assert lq(st) == [1] and st.request_ids.tolist() == [0]
    s.complete()
    s2 = sched(1024, blocks=4, mb=64)
    s2.add(0, 64, 3)
    assert lq(s2.next_step()) == [64]
    s2.complete()
    with pytest.raises(B.HybridAttnError):
        s2.next_step()  # the pool is full and the request needs a new page


def test_max_seqs_caps_segments_per_step():
    s = sched(1024, max_seqs=4)
    for r in range(10):
        s.add(r, 5, 1)
    st = s.next_step()
    assert st.num_seqs == 4 and st.request_ids.tolist() == [0, 1, 2, 3]


def test_argument_errors():
    from chunked_prefill_mixed_hybrid_amd.scheduler import StepScheduler
    with pytest.raises(ValueError):
        StepScheduler(0, 10, 10)
    s = sched(64, mb=4)
    with pytest.raises(B.HybridAttnError):
        s.add(0, 0, 1)
    with pytest.raises(B.HybridAttnError):
        s.add(0, 60, 6)  # 65 tokens need 5 pages > 4
    s.add(0, 60, 5)
    with pytest.raises(B.HybridAttnError):
        s.add(0, 1, 1)  # live duplicate id
    s.next_step()
    with pytest.raises(B.HybridAttnError):
        s.add(1, 1, 1)  # between next_step and complete
    with pytest.raises(B.HybridAttnError):
        s.next_step()
    s.complete()
    with pytest.raises(B.HybridAttnError):
        s.complete()


def request_values(rid, n, hq, hkv, d, seed=11):
    rng = np.random.default_rng([seed, rid])
    return (rng.standard_normal((n, hq, d)).astype(np.float32),
            rng.standard_normal((n, hkv, d)).astype(np.float32),
            rng.standard_normal((n, hkv, d)).astype(np.float32))


def test_scheduled_steps_match_each_request_in_one_piece(orc):
    """Oracle over the scheduled steps (shared pool, mixed segments) equals the
    oracle over each request's whole sequence in one step, bit for bit in fp64:
    the scheduler's metadata (positions, pages, slots, lengths) is exact."""
    hq, hkv, d = 2, 1, 16
    reqs = {0: (37, 5), 1: (150, 3), 2: (300, 8), 3: (64, 2), 4: (1, 4)}
    vals = {r: request_values(r, p + g - 1, hq, hkv, d) for r, (p, g) in reqs.items()}
    nb, mb = 96, 32
    s = sched(128, blocks=nb, mb=mb)
    for r, (p, g) in reqs.items():
        s.add(r, p, g)
    kc = np.full((nb, PAGE, hkv, d), np.nan, np.float32)
    vc = kc.copy()
    got = {r: {} for r in reqs}
    for st in run_all_steps(s):
        rows = [(int(r), int(f) + i) for r, f, n in
                zip(st.request_ids, st.first_pos, np.diff(st.cu_seqlens_q)) for i in range(n)]
        q = np.stack([vals[r][0][p] for r, p in rows])
        k = np.stack([vals[r][1][p] for r, p in rows])
        v = np.stack([vals[r][2][p] for r, p in rows])
        orc.append(k, v, st.slot_mapping, kc, vc)
        out = orc.attention(q, kc, vc, st.cu_seqlens_q, st.seqlens_k, st.block_table)
        for (r, p), o in zip(rows, out):
            got[r][p] = o
    for r, (p, g) in reqs.items():
        n = p + g - 1
        q, k, v = vals[r]
        npages = -(-n // PAGE)
        bt = np.arange(npages, dtype=np.int32)[None]
        kc1 = np.full((npages, PAGE, hkv, d), np.nan, np.float32)
        vc1 = kc1.copy()
        orc.append(k, v, np.arange(n, dtype=np.int32), kc1, vc1)
        ref = orc.attention(q, kc1, vc1, np.array([0, n], np.int32), np.array([n], np.int32), bt)
        assert sorted(got[r]) == list(range(n))
        assert np.array_equal(np.stack([got[r][i] for i in range(n)]), ref), r


def run_all_steps(s):
    while True:
        st = s.next_step()
        if st is None:
            return
        yield st
        s.complete()
