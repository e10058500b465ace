"""Thin ctypes binding of libhybridattn.so (argument marshalling only).

Every step of the mixed attention step runs in the library's HIP kernels;
PyTorch only provides device memory and the stream.  The library must have
been built (python -m chunked_prefill_mixed_hybrid_amd.build); a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libhybridattn.so"

HA_OK, HA_ERR_INVALID_ARGUMENT, HA_ERR_UNSUPPORTED, HA_ERR_WORKSPACE_TOO_SMALL, HA_ERR_HIP = range(5)
HA_DTYPE_F32, HA_DTYPE_BF16 = 0, 1

EXPORTED = ("ha_status_string", "paged_kv_append", "hybrid_attn_workspace_size", "hybrid_attn_fwd",
            "hybrid_attn_fwd_two_launch", "varlen_attn_fwd", "hybrid_step_fwd",
            "hybrid_step_fwd_noalloc")


class HybridAttnError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {text} ({status})")
        self.status = status


_lib = None


def load(path: Path | str | None = None) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} not found: build it with `python -m chunked_prefill_mixed_hybrid_amd.build`")
    # torch first: the library must bind to the HIP runtime torch loads (the
    # ROCm torch wheel carries its own); loaded before it, the library would
    # pull in a second runtime that cannot see torch's memory or streams
    import torch  # noqa: F401
    lib = ctypes.CDLL(str(p))
    i32, vp, i32p = ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    lib.ha_status_string.argtypes = [ctypes.c_int]
    lib.ha_status_string.restype = ctypes.c_char_p
    lib.paged_kv_append.argtypes = [vp, vp, i32p, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.paged_kv_append.restype = ctypes.c_int
    lib.hybrid_attn_workspace_size.argtypes = [i32] * 5
    lib.hybrid_attn_workspace_size.restype = ctypes.c_size_t
    lib.hybrid_attn_fwd.argtypes = ([vp, vp, vp, i32p, i32p, i32p, vp] + [i32] * 10 +
                                    [ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t, vp])
    lib.hybrid_attn_fwd.restype = ctypes.c_int
    lib.hybrid_attn_fwd_two_launch.argtypes = ([vp, vp, vp, i32p, i32p, i32p, vp] + [i32] * 10 +
                                               [ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t,
                                                i32, vp])
    lib.hybrid_attn_fwd_two_launch.restype = ctypes.c_int
    lib.varlen_attn_fwd.argtypes = ([vp, vp, vp, i32p, i32p, vp] + [i32] * 8 +
                                    [ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t, vp])
    lib.varlen_attn_fwd.restype = ctypes.c_int
    lib.hybrid_step_fwd.argtypes = ([vp, vp, i32p, vp, vp, vp, i32p, i32p, i32p, vp] + [i32] * 10 +
                                    [ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t, vp])
    lib.hybrid_step_fwd.restype = ctypes.c_int
    lib.hybrid_step_fwd_noalloc.argtypes = ([vp, vp, i32p, vp, vp, vp, i32p, i32p, i32p, vp] +
                                            [i32] * 10 + [ctypes.c_float, ctypes.c_int, vp])
    lib.hybrid_step_fwd_noalloc.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().ha_status_string(status).decode()


def _check(fn, status):
    if status != HA_OK:
        raise HybridAttnError(fn, status, status_string(status))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return HA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return HA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _scale(sm_scale) -> float:
    """sm_scale as passed to the library: 0 asks the library for its default."""
    return 0.0 if sm_scale is None else float(sm_scale)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def paged_kv_append(key, value, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """key/value [T, Hkv, D] -> k_cache/v_cache [NB, P, Hkv, D] at slot_mapping[T]."""
    import torch
    t, hkv, d = key.shape
    nb, p, hkv2, d2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (hkv, d) != (hkv2, d2):
        raise ValueError("paged_kv_append: shape mismatch")
    if slot_mapping.shape != (t,):
        raise ValueError("paged_kv_append: slot_mapping must be [T]")
    dt = key.dtype
    st = load().paged_kv_append(_dev(key, "key", dt), _dev(value, "value", dt),
                                _dev(slot_mapping, "slot_mapping", torch.int32),
                                _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
                                t, hkv, d, p, nb, _dtype_code(key), _stream(stream))
    _check("paged_kv_append", st)


def workspace_size(num_seqs, total_q, max_seqlen_k, num_heads, head_dim) -> int:
    return int(load().hybrid_attn_workspace_size(num_seqs, total_q, max_seqlen_k, num_heads, head_dim))


def alloc_workspace(num_seqs, total_q, max_seqlen_k, num_heads, head_dim, device="cuda"):
    import torch
    n = workspace_size(num_seqs, total_q, max_seqlen_k, num_heads, head_dim)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def hybrid_attn_fwd(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, max_seqlen_q,
                    max_seqlen_k, out=None, sm_scale=None, workspace=None, stream=None):
    """One fused varlen paged attention forward (causal, right-aligned)."""
    return _attn("hybrid_attn_fwd", q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                 max_seqlen_q, max_seqlen_k, out, sm_scale, workspace, stream, ())


def hybrid_attn_fwd_two_launch(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                               max_seqlen_q, max_seqlen_k, out=None, sm_scale=None,
                               workspace=None, two_streams=False, stream=None):
    """The same computation with the chunk and decode roles in two launches
    (back to back, or concurrently on two streams): a comparison baseline."""
    return _attn("hybrid_attn_fwd_two_launch", q, k_cache, v_cache, cu_seqlens_q, seqlens_k,
                 block_table, max_seqlen_q, max_seqlen_k, out, sm_scale, workspace, stream,
                 (1 if two_streams else 0,))


def hybrid_step_fwd(key, value, slot_mapping, q, k_cache, v_cache, cu_seqlens_q, seqlens_k,
                    block_table, max_seqlen_q, max_seqlen_k, out=None, sm_scale=None,
                    workspace=None, stream=None):
    """One whole mixed step: paged_kv_append(key, value, slot_mapping) into the
    pools, then hybrid_attn_fwd -- the same result, with the append and the
    planner sharing a launch when the step allows it."""
    import torch
    t, hq, d = q.shape
    nb, p, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or key.shape != (t, hkv, d) or value.shape != key.shape:
        raise ValueError("hybrid_step_fwd: shape mismatch")
    b = seqlens_k.shape[0]
    if (cu_seqlens_q.shape != (b + 1,) or block_table.dim() != 2 or block_table.shape[0] != b
            or slot_mapping.shape != (t,)):
        raise ValueError("hybrid_step_fwd: metadata shapes")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(b, t, max_seqlen_k, hq, d, device=q.device)
    scale = _scale(sm_scale)
    dt = q.dtype
    st = load().hybrid_step_fwd(
        _dev(key, "key", dt), _dev(value, "value", dt),
        _dev(slot_mapping, "slot_mapping", torch.int32), _dev(q, "q", dt),
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqlens_k, "seqlens_k", torch.int32),
        _dev(block_table, "block_table", torch.int32), _dev(out, "out", dt),
        b, t, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, p, nb, block_table.shape[1],
        scale, _dtype_code(q), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream))
    _check("hybrid_step_fwd", st)
    return out


def hybrid_step_fwd_noalloc(key, value, slot_mapping, q, k_cache, v_cache, cu_seqlens_q,
                            seqlens_k, block_table, max_seqlen_q, max_seqlen_k, out,
                            sm_scale=None, stream=None):
    """hybrid_step_fwd with the library's own device scratch array as its
    workspace: the call allocates no device memory (`out` is the caller's)."""
    import torch
    t, hq, d = q.shape
    nb, p, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or key.shape != (t, hkv, d) or value.shape != key.shape:
        raise ValueError("hybrid_step_fwd_noalloc: shape mismatch")
    b = seqlens_k.shape[0]
    if (cu_seqlens_q.shape != (b + 1,) or block_table.dim() != 2 or block_table.shape[0] != b
            or slot_mapping.shape != (t,) or out.shape != q.shape):
        raise ValueError("hybrid_step_fwd_noalloc: metadata or output shapes")
    dt = q.dtype
    st = load().hybrid_step_fwd_noalloc(
        _dev(key, "key", dt), _dev(value, "value", dt),
        _dev(slot_mapping, "slot_mapping", torch.int32), _dev(q, "q", dt),
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqlens_k, "seqlens_k", torch.int32),
        _dev(block_table, "block_table", torch.int32), _dev(out, "out", dt),
        b, t, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, p, nb, block_table.shape[1],
        _scale(sm_scale), _dtype_code(q), _stream(stream))
    _check("hybrid_step_fwd_noalloc", st)
    return out


def varlen_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, out=None,
                    sm_scale=None, workspace=None, stream=None):
    """The same attention over K/V packed per segment: segment b's keys are rows
    cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1 of k and v [total_k, Hkv, D]."""
    import torch
    t, hq, d = q.shape
    tk, hkv, d2 = k.shape
    if d2 != d or v.shape != k.shape:
        raise ValueError("varlen_attn_fwd: shape mismatch")
    b = cu_seqlens_k.shape[0] - 1
    if cu_seqlens_q.shape != (b + 1,):
        raise ValueError("varlen_attn_fwd: metadata shapes")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(b, t, max_seqlen_k, hq, d, device=q.device)
    scale = _scale(sm_scale)
    dt = q.dtype
    st = load().varlen_attn_fwd(
        _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), _dev(out, "out", dt),
        b, t, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, scale, _dtype_code(q),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check("varlen_attn_fwd", st)
    return out


def _attn(fn, q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, max_seqlen_q,
          max_seqlen_k, out, sm_scale, workspace, stream, extra):
    import torch
    t, hq, d = q.shape
    nb, p, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError(f"{fn}: shape mismatch")
    b = seqlens_k.shape[0]
    if cu_seqlens_q.shape != (b + 1,) or block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError(f"{fn}: metadata shapes")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(b, t, max_seqlen_k, hq, d, device=q.device)
    scale = _scale(sm_scale)
    dt = q.dtype
    st = getattr(load(), fn)(
        _dev(q, "q", dt), _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqlens_k, "seqlens_k", torch.int32),
        _dev(block_table, "block_table", torch.int32), _dev(out, "out", dt),
        b, t, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, p, nb, block_table.shape[1],
        scale, _dtype_code(q), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        *extra, _stream(stream))
    _check(fn, st)
    return out
