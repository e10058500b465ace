"""ctypes wrapper of the token-budget step generator (include/ha_scheduler.h).

    s = StepScheduler(budget=2048, num_blocks=4096, max_blocks_per_seq=1024)
    s.add(request_id=0, prompt_len=10000, max_new_tokens=4)
    while (step := s.next_step()) is not None:
        ...  # run paged_kv_append + hybrid_attn_fwd with step's metadata
        finished = s.complete()

Argument marshalling only: the policy lives in csrc/scheduler.cpp.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import binding as B

EXPORTED = ("ha_sched_create", "ha_sched_destroy", "ha_sched_add_request", "ha_sched_next_step",
            "ha_sched_complete_step", "ha_sched_num_unfinished", "ha_sched_free_blocks")


class StepShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
                ("num_decodes", ctypes.c_int32), ("num_sampling", ctypes.c_int32)]


_configured = set()


def _lib():
    lib = B.load()
    if id(lib) in _configured:
        return lib
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.ha_sched_create.argtypes = [i32, i32, i32, i32]
    lib.ha_sched_create.restype = vp
    lib.ha_sched_destroy.argtypes = [vp]
    lib.ha_sched_destroy.restype = None
    lib.ha_sched_add_request.argtypes = [vp, i64, i32, i32]
    lib.ha_sched_add_request.restype = ctypes.c_int
    lib.ha_sched_next_step.argtypes = [vp, ctypes.POINTER(StepShape)] + [vp] * 6 + [i32, i32]
    lib.ha_sched_next_step.restype = ctypes.c_int
    lib.ha_sched_complete_step.argtypes = [vp, vp, i32, vp]
    lib.ha_sched_complete_step.restype = ctypes.c_int
    lib.ha_sched_num_unfinished.argtypes = [vp]
    lib.ha_sched_num_unfinished.restype = i32
    lib.ha_sched_free_blocks.argtypes = [vp]
    lib.ha_sched_free_blocks.restype = i32
    _configured.add(id(lib))
    return lib


@dataclass
class Step:
    """Metadata of one planned step (host arrays, int32 unless noted)."""
    cu_seqlens_q: np.ndarray   # [B+1]
    seqlens_k: np.ndarray      # [B]
    block_table: np.ndarray    # [B, max_blocks_per_seq]
    slot_mapping: np.ndarray   # [T]
    request_ids: np.ndarray    # int64 [B]
    first_pos: np.ndarray      # [B]: position of each segment's first query row
    max_seqlen_q: int
    max_seqlen_k: int
    num_decodes: int
    num_sampling: int

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens_k)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])


class StepScheduler:
    """Running requests first, then the waiting queue, within a token budget."""

    def __init__(self, budget: int, num_blocks: int, max_blocks_per_seq: int,
                 long_prefill_token_threshold: int = 0, max_seqs: int = 1024):
        self._lib = _lib()
        self._h = self._lib.ha_sched_create(budget, long_prefill_token_threshold, num_blocks,
                                            max_blocks_per_seq)
        if not self._h:
            raise ValueError("ha_sched_create: invalid arguments")
        self.budget, self.max_blocks, self.max_seqs = budget, max_blocks_per_seq, max_seqs
        self._cu = np.zeros(max_seqs + 1, np.int32)
        self._sk = np.zeros(max_seqs, np.int32)
        self._bt = np.zeros((max_seqs, max_blocks_per_seq), np.int32)
        self._sm = np.zeros(budget, np.int32)
        self._ids = np.zeros(max_seqs, np.int64)
        self._fp = np.zeros(max_seqs, np.int32)
        self._fin = np.zeros(max_seqs, np.int64)

    def close(self):
        if self._h:
            self._lib.ha_sched_destroy(self._h)
            self._h = None

    __del__ = close

    def add(self, request_id: int, prompt_len: int, max_new_tokens: int):
        st = self._lib.ha_sched_add_request(self._h, request_id, prompt_len, max_new_tokens)
        if st != B.HA_OK:
            raise B.HybridAttnError("ha_sched_add_request", st, B.status_string(st))

    def next_step(self) -> Step | None:
        """Plans the next step; None when every request has finished."""
        sh = StepShape()
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        st = self._lib.ha_sched_next_step(self._h, ctypes.byref(sh), p(self._cu), p(self._sk),
                                          p(self._bt), p(self._sm), p(self._ids), p(self._fp),
                                          self.max_seqs, self.budget)
        if st != B.HA_OK:
            raise B.HybridAttnError("ha_sched_next_step", st, B.status_string(st))
        b = sh.num_seqs
        if b == 0:
            return None
        return Step(self._cu[:b + 1].copy(), self._sk[:b].copy(), self._bt[:b].copy(),
                    self._sm[:sh.total_q].copy(), self._ids[:b].copy(), self._fp[:b].copy(),
                    sh.max_seqlen_q, sh.max_seqlen_k, sh.num_decodes, sh.num_sampling)

    def complete(self) -> list:
        """Marks the planned step as run; returns the ids of finished requests."""
        n = ctypes.c_int32(0)
        st = self._lib.ha_sched_complete_step(self._h, self._fin.ctypes.data_as(ctypes.c_void_p),
                                              len(self._fin), ctypes.byref(n))
        if st != B.HA_OK:
            raise B.HybridAttnError("ha_sched_complete_step", st, B.status_string(st))
        return self._fin[:min(n.value, len(self._fin))].tolist()

    @property
    def unfinished(self) -> int:
        return int(self._lib.ha_sched_num_unfinished(self._h))

    @property
    def free_blocks(self) -> int:
        return int(self._lib.ha_sched_free_blocks(self._h))
