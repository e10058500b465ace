"""The step generator driving the HIP path: a multi-request trace scheduled under
a token budget (running first, waiting fill; wangyu.me chunked-prefill page,
section on the vLLM implementation), every step run through paged_kv_append and
hybrid_attn_fwd on one shared page pool, against the oracle step by step;
afterwards the pools must be byte-identical and each request's rows must agree
with that request run alone in one step (chunk invariance across requests)."""
import numpy as np
import pytest

from chunked_prefill_mixed_hybrid_amd import binding as B
from chunked_prefill_mixed_hybrid_amd import workload as W
import gpu_support as G

pytestmark = pytest.mark.gpu

PAGE = 16
TRACES = [
    # (requests {id: (prompt, new tokens)}, heads, kv heads, dim, dtype, budget, threshold)
    ({0: (3000, 4), 1: (700, 6), 2: (1500, 3), 3: (64, 9), 4: (2100, 2), 5: (1, 5)},
     8, 8, 128, W.BF16, 1024, 0),
    ({0: (2500, 3), 1: (130, 4), 2: (900, 2), 3: (77, 7)}, 4, 2, 64, W.F32, 512, 300),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("case", range(len(TRACES)))
def test_scheduled_trace_on_gpu(case, orc):
    import torch
    from chunked_prefill_mixed_hybrid_amd.scheduler import StepScheduler
    reqs, hq, hkv, d, dt, budget, thr = TRACES[case]
    vals = {r: W.request_values(r, p + g - 1, hq, hkv, d, dt, seed=case) for r, (p, g) in reqs.items()}
    nb, mb = 1024, 256
    s = StepScheduler(budget, nb, mb, long_prefill_token_threshold=thr)
    for r, (p, g) in reqs.items():
        s.add(r, p, g)
    nanv = W.nan_value(dt)
    kc_h = np.full((nb, PAGE, hkv, d), nanv)
    vc_h = kc_h.copy()
    kc, vc = _dev(kc_h), _dev(vc_h)
    got = {r: {} for r in reqs}
    n_steps = 0
    while (st := s.next_step()) is not None:
        rows, q, k, v = W.step_tokens(st.request_ids, st.first_pos, st.cu_seqlens_q, vals)
        G.note(f"scheduled trace {case} step {n_steps}: {st.num_seqs} segments, {st.total_q} rows")
        B.paged_kv_append(_dev(k), _dev(v), _i32(st.slot_mapping), kc, vc)
        out = B.hybrid_attn_fwd(_dev(q), kc, vc, _i32(st.cu_seqlens_q), _i32(st.seqlens_k),
                                _i32(st.block_table), st.max_seqlen_q, st.max_seqlen_k)
        torch.cuda.synchronize()
        orc.append(k, v, st.slot_mapping, kc_h, vc_h)
        ref = orc.attention(q, kc_h, vc_h, st.cu_seqlens_q, st.seqlens_k, st.block_table)
        o = G.to_f64(out)
        G.compare(o, ref, dt, f"trace {case} step {n_steps}")
        for (r, p), row in zip(rows, o):
            got[r][p] = row
        s.complete()
        n_steps += 1
    assert n_steps > 5 and s.unfinished == 0 and s.free_blocks == nb
    assert W.to_host_array(kc).tobytes() == kc_h.tobytes()
    assert W.to_host_array(vc).tobytes() == vc_h.tobytes()
    # each request alone, in one step, on the GPU: the same rows within tolerance
    for r, (p, g) in reqs.items():
        n = p + g - 1
        q, k, v = vals[r]
        npg = -(-n // PAGE)
        kc1 = _dev(np.full((npg, PAGE, hkv, d), nanv))
        vc1 = _dev(np.full((npg, PAGE, hkv, d), nanv))
        B.paged_kv_append(_dev(k), _dev(v), _i32(np.arange(n)), kc1, vc1)
        one = B.hybrid_attn_fwd(_dev(q), kc1, vc1, _i32([0, n]), _i32([n]),
                                _i32(np.arange(npg)[None]), n, n)
        torch.cuda.synchronize()
        assert sorted(got[r]) == list(range(n))
        G.compare(np.stack([got[r][i] for i in range(n)]), G.to_f64(one), dt, f"request {r} alone")
