"""Seeded synthetic inputs for mixed chunked-prefill steps.

This module only builds inputs: segment shapes, the per-step metadata arrays
(cu_seqlens_q, seqlens_k, block_table, slot_mapping), random Q/K/V values and
NaN poison in cache slots no kernel may read.  It contains none of the
attention arithmetic.  Both the HIP path's tests/benchmark and the CPU oracle
consume what it produces.

Shapes follow the source pages' workloads:
  * worked example: decode A (120 history + 1), decode B (45 + 1), prefill C
    (10000-token prompt, 8192 done, last 1808) -- "大语言模型推理优化（二）：
    Chunked Prefill" (wangyu.me), section "组装长序列" / "记录 KV Cache 的长度";
  * 2 chunks of 512 + 30 decodes -- lpnh.cn FlashAttention/FlashInfer article,
    section 2 (mixed batch example);
  * decode-heavy, long-context (32K-128K) and budget-2048 steps -- kwkr.cn
    Triton article intro (32K ~ 128K prompts) and the wangyu.me page's token
    budget section (max_num_batched_tokens = 2048);
  * 10000-token prompt prefilled as 4 x 2048 + 1808 vs one step -- wangyu.me
    page, sections "Chunked Prefill 的原理" and "Chunked Prefill 的注意力计算".
Page size is 16 tokens (kwkr.cn Triton article launcher constants).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16
F32, BF16 = "f32", "bf16"


@dataclass
class StepSpec:
    """One step: packed segments (Lq, Lk) in packing order, head shape, dtype."""
    name: str
    segments: list  # list of (Lq, Lk); Lk counts history + this step's new tokens
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    page_size: int = PAGE_SIZE
    spare_blocks: int = 8  # pages no segment owns (poisoned)

    @property
    def total_q(self) -> int:
        return int(sum(lq for lq, _ in self.segments))


@dataclass
class StepMeta:
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    seqlens_k: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_blocks], -1 past each segment's pages
    slot_mapping: np.ndarray  # int32 [T]
    num_blocks: int
    page_size: int
    max_seqlen_q: int
    max_seqlen_k: int
    poison_slots: np.ndarray = field(default=None)  # int64 slots to fill with NaN

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens_k)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]


def _decodes(rng, n, lo, hi):
    hist = rng.integers(lo, hi, n, endpoint=True)
    return [(1, int(h) + 1) for h in hist]


CONFIGS = ("1", "2", "3", "4", "5", "5a", "5b")


def config_spec(config, seed: int = 0) -> tuple:
    """(StepSpec, rng) for workload configs 1..5 (5 or "5a" = the budget-2048
    step; "5b" = the 10000-token prompt of the chunk-equivalence run prefilled
    in one step, 64 heads x 128, bf16).

    The returned rng has drawn the decode histories and is then used for the
    block-id permutation, so the whole step follows from (config, seed)."""
    rng = np.random.default_rng(seed)
    config = str(config)
    if config == "5b":
        return StepSpec("full_prefill_10000_64x128", [(10000, 10000)], 64, 64, 128, BF16), rng
    config = 5 if config == "5a" else int(config)
    if config == 1:
        segs = [(1, 121), (1, 46), (1808, 10000)]
        return StepSpec("worked_example", segs, 2, 2, 64, F32), rng
    if config == 2:
        segs = [(512, 512), (512, 2048)] + _decodes(rng, 30, 512, 4096)
        return StepSpec("mixed_2x512_30dec", segs, 32, 32, 128, BF16), rng
    if config == 3:
        segs = [(512, 2560)] + _decodes(rng, 256, 1024, 32768)
        return StepSpec("decode_heavy_512_256dec", segs, 32, 32, 128, BF16), rng
    if config == 4:
        segs = [(1024, 131072)] + _decodes(rng, 64, 8192, 131072)
        return StepSpec("long_context_1024at130K_64dec", segs, 32, 32, 128, BF16), rng
    if config == 5:
        segs = _decodes(rng, 64, 1024, 16384) + [(1984, 10176)]
        return StepSpec("budget2048_64dec_1984chunk", segs, 64, 64, 128, BF16), rng
    raise ValueError(f"unknown config {config}")


def chunked_prompt_steps(prompt_len=10000, chunk=2048):
    """(Lq, Lk) of each step when a prompt is prefilled chunk by chunk."""
    steps, done = [], 0
    while done < prompt_len:
        n = min(chunk, prompt_len - done)
        done += n
        steps.append((n, done))
    return steps


def build_meta(spec: StepSpec, rng: np.random.Generator) -> StepMeta:
    """Metadata as a model runner would build it: every segment owns
    ceil(Lk/P) pages whose physical ids come from a random permutation of the
    pool (plus a few spare pages nobody owns); the step's new tokens are the
    last Lq positions of each segment and land in the slot their position maps
    to through the segment's block-table row."""
    p = spec.page_size
    lqs = np.array([lq for lq, _ in spec.segments], dtype=np.int64)
    lks = np.array([lk for _, lk in spec.segments], dtype=np.int64)
    if np.any(lqs > lks):
        raise ValueError("a segment has more queries than keys")
    pages = (lks + p - 1) // p
    used = int(pages.sum())
    nb = used + spec.spare_blocks
    perm = rng.permutation(nb).astype(np.int64)
    max_blocks = max(1, int(pages.max()) if len(pages) else 1)
    bt = np.full((len(lks), max_blocks), -1, dtype=np.int64)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    spare = perm[off:]

    cu = np.zeros(len(lqs) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lqs)
    slot = np.empty(int(cu[-1]), dtype=np.int64)
    tails = []
    for b in range(len(lks)):
        pos = np.arange(lks[b] - lqs[b], lks[b])
        slot[cu[b]:cu[b + 1]] = bt[b, pos // p] * p + pos % p
        tail = np.arange(lks[b], pages[b] * p)
        tails.append(bt[b, tail // p] * p + tail % p)
    spare_slots = (spare[:, None] * p + np.arange(p)[None, :]).reshape(-1)
    poison = np.concatenate([slot] + tails + [spare_slots]).astype(np.int64)
    return StepMeta(cu.astype(np.int32), lks.astype(np.int32), bt.astype(np.int32),
                    slot.astype(np.int32), nb, p, int(lqs.max()) if len(lqs) else 0,
                    int(lks.max()) if len(lks) else 0, poison)


def make_step(config, seed: int = 0):
    spec, rng = config_spec(config, seed)
    return spec, build_meta(spec, rng)


def custom_step(segments, num_heads, num_kv_heads, head_dim, dtype, seed=0, spare_blocks=8,
                page_size=PAGE_SIZE):
    rng = np.random.default_rng(seed)
    spec = StepSpec("custom", list(segments), num_heads, num_kv_heads, head_dim, dtype,
                    page_size, spare_blocks)
    return spec, build_meta(spec, rng)


# ---------------------------------------------------------------------------------
# values

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, as raw uint16 bits (via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == F32 else f32_to_bf16_bits(x)


def nan_value(dtype: str):
    return np.float32(np.nan) if dtype == F32 else np.uint16(0x7FC0)


@dataclass
class HostStep:
    spec: StepSpec
    meta: StepMeta
    q: np.ndarray  # [T, Hq, D]
    key: np.ndarray  # [T, Hkv, D]
    value: np.ndarray
    k_cache: np.ndarray  # [NB, P, Hkv, D], history filled, everything else NaN
    v_cache: np.ndarray


def host_values(spec: StepSpec, meta: StepMeta, seed: int = 0, poison: bool = True) -> HostStep:
    """N(0,1) values drawn with numpy on the host (small steps, CPU tests)."""
    rng = np.random.default_rng([seed, 1])
    t, hq, hkv, d, p = meta.total_q, spec.num_heads, spec.num_kv_heads, spec.head_dim, meta.page_size
    q = _store(rng.standard_normal((t, hq, d), dtype=np.float32), spec.dtype)
    key = _store(rng.standard_normal((t, hkv, d), dtype=np.float32), spec.dtype)
    value = _store(rng.standard_normal((t, hkv, d), dtype=np.float32), spec.dtype)
    kc = _store(rng.standard_normal((meta.num_blocks, p, hkv, d), dtype=np.float32), spec.dtype)
    vc = _store(rng.standard_normal((meta.num_blocks, p, hkv, d), dtype=np.float32), spec.dtype)
    if poison:
        nanv = nan_value(spec.dtype)
        for c in (kc, vc):
            c.reshape(-1, hkv * d)[meta.poison_slots] = nanv
    return HostStep(spec, meta, q, key, value, kc, vc)


def request_values(request_id: int, n_tokens: int, num_heads: int, num_kv_heads: int,
                   head_dim: int, dtype: str, seed: int = 0):
    """q [n, Hq, D], k and v [n, Hkv, D] of every token of one request (prompt and
    generated tokens), drawn per request so that whichever step schedules a
    token sees the same bytes."""
    rng = np.random.default_rng([seed, 2, int(request_id)])
    q = _store(rng.standard_normal((n_tokens, num_heads, head_dim), dtype=np.float32), dtype)
    k = _store(rng.standard_normal((n_tokens, num_kv_heads, head_dim), dtype=np.float32), dtype)
    v = _store(rng.standard_normal((n_tokens, num_kv_heads, head_dim), dtype=np.float32), dtype)
    return q, k, v


def step_tokens(request_ids, first_pos, cu_seqlens_q, values):
    """(request, position) of every query row of a scheduled step, and the q /
    key / value rows gathered from per-request `values` {id: (q, k, v)}."""
    n = np.diff(np.asarray(cu_seqlens_q))
    rows = [(int(r), int(f) + i) for r, f, c in zip(request_ids, first_pos, n) for i in range(c)]
    q = np.stack([values[r][0][p] for r, p in rows])
    k = np.stack([values[r][1][p] for r, p in rows])
    v = np.stack([values[r][2][p] for r, p in rows])
    return rows, q, k, v


def torch_dtype(dtype: str):
    import torch
    return torch.float32 if dtype == F32 else torch.bfloat16


def fill_randn_(t, gen, slab_elems: int = 1 << 28):
    """Fill a (possibly huge) tensor with N(0,1) in slabs of <= 1 GiB fp32."""
    import torch
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, slab_elems):
        e = min(n, s + slab_elems)
        tmp = torch.randn(e - s, generator=gen, device=t.device, dtype=torch.float32)
        flat[s:e].copy_(tmp)
        del tmp
    return t


@dataclass
class DeviceStep:
    spec: StepSpec
    meta: StepMeta
    q: object
    key: object
    value: object
    k_cache: object
    v_cache: object
    cu_seqlens_q: object
    seqlens_k: object
    block_table: object
    slot_mapping: object


def device_values(spec: StepSpec, meta: StepMeta, seed: int = 0, device="cuda",
                  poison: bool = True) -> DeviceStep:
    """N(0,1) values drawn on the device with a seeded torch generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = torch_dtype(spec.dtype)
    t, hq, hkv, d, p = meta.total_q, spec.num_heads, spec.num_kv_heads, spec.head_dim, meta.page_size
    q = fill_randn_(torch.empty((t, hq, d), dtype=dt, device=device), gen)
    key = fill_randn_(torch.empty((t, hkv, d), dtype=dt, device=device), gen)
    value = fill_randn_(torch.empty((t, hkv, d), dtype=dt, device=device), gen)
    kc = fill_randn_(torch.empty((meta.num_blocks, p, hkv, d), dtype=dt, device=device), gen)
    vc = fill_randn_(torch.empty((meta.num_blocks, p, hkv, d), dtype=dt, device=device), gen)
    if poison:
        idx = torch.from_numpy(meta.poison_slots).to(device)
        for c in (kc, vc):
            c.view(-1, hkv * d).index_fill_(0, idx, float("nan"))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)  # noqa: E731
    return DeviceStep(spec, meta, q, key, value, kc, vc, i32(meta.cu_seqlens_q),
                      i32(meta.seqlens_k), i32(meta.block_table), i32(meta.slot_mapping))


def to_device(hs: HostStep, device="cuda") -> DeviceStep:
    """Upload a host-generated step (same bytes) to the device."""
    import torch

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)  # noqa: E731
    m = hs.meta
    return DeviceStep(hs.spec, m, up(hs.q), up(hs.key), up(hs.value), up(hs.k_cache),
                      up(hs.v_cache), i32(m.cu_seqlens_q), i32(m.seqlens_k),
                      i32(m.block_table), i32(m.slot_mapping))


def to_host_array(t) -> np.ndarray:
    """torch tensor (any device) -> numpy; bf16 becomes raw uint16 bits."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
