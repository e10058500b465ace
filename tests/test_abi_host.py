"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/hybrid_attn.h declares, sizes workspaces, and rejects
bad arguments with the documented status codes before touching the GPU."""
import ctypes
import re
from pathlib import Path

import pytest

from chunked_prefill_mixed_hybrid_amd import binding as B

HEADERS = sorted((Path(__file__).resolve().parent.parent / "include").glob("*.h"))


@pytest.fixture(scope="module")
def lib():
    if not B.LIB_PATH.exists():
        from chunked_prefill_mixed_hybrid_amd import build
        build.build()
    return B.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\(", text, re.M))
    return sorted(names)


def test_headers_declare_the_abi():
    from chunked_prefill_mixed_hybrid_amd import scheduler
    assert len(HEADERS) == 2
    assert declared_functions() == sorted(B.EXPORTED + scheduler.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in enumerate(["HA_OK", "HA_ERR_INVALID_ARGUMENT", "HA_ERR_UNSUPPORTED",
                                 "HA_ERR_WORKSPACE_TOO_SMALL", "HA_ERR_HIP"]):
        assert B.status_string(code) == name


def test_workspace_size_grows_with_bounds(lib):
    a = B.workspace_size(32, 1054, 4097, 32, 128)
    assert a > 0 and a % 256 == 0
    assert B.workspace_size(64, 1054, 4097, 32, 128) > a
    assert B.workspace_size(32, 1054, 4097, 64, 128) > a
    assert B.workspace_size(0, 10, 10, 1, 64) == 0


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails host-side


def fwd(lib, entry="hybrid_attn_fwd", **kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, cu=FAKE, sk=FAKE, bt=FAKE, out=FAKE, B=3, T=1810,
                mq=1808, mk=10000, H=2, Hkv=2, D=64, P=16, NB=644, MB=625, scale=0.125,
                dt=B.HA_DTYPE_F32, ws=FAKE, wsb=1 << 30)
    args.update(kw)
    extra = [args.pop("two_streams")] if "two_streams" in args else []
    if entry == "hybrid_attn_fwd_two_launch" and not extra:
        extra = [0]
    return getattr(lib, entry)(*args.values(), *extra, None)


@pytest.mark.parametrize("entry", ["hybrid_attn_fwd", "hybrid_attn_fwd_two_launch"])
def test_fwd_argument_errors(lib, entry):
    fwd = lambda lib, **kw: globals()["fwd"](lib, entry, **kw)  # noqa: E731
    assert fwd(lib, Hkv=3) == B.HA_ERR_INVALID_ARGUMENT  # 2 % 3 != 0
    assert fwd(lib, mq=20000) == B.HA_ERR_INVALID_ARGUMENT  # max_seqlen_q > max_seqlen_k
    assert fwd(lib, B=0) == B.HA_ERR_INVALID_ARGUMENT
    assert fwd(lib, q=None) == B.HA_ERR_INVALID_ARGUMENT
    assert fwd(lib, bt=None) == B.HA_ERR_INVALID_ARGUMENT
    assert fwd(lib, ws=ctypes.c_void_p(0x100010)) == B.HA_ERR_INVALID_ARGUMENT  # not 256-aligned
    assert fwd(lib, D=96) == B.HA_ERR_UNSUPPORTED
    assert fwd(lib, P=32) == B.HA_ERR_UNSUPPORTED
    assert fwd(lib, dt=7) == B.HA_ERR_UNSUPPORTED
    need = B.workspace_size(3, 1810, 10000, 2, 64)
    assert fwd(lib, wsb=need - 1) == B.HA_ERR_WORKSPACE_TOO_SMALL
    assert fwd(lib, T=0, wsb=need) == B.HA_OK  # nothing to do, nothing enqueued
    if entry == "hybrid_attn_fwd_two_launch":
        assert fwd(lib, T=0, wsb=need, two_streams=1) == B.HA_OK
        assert fwd(lib, wsb=need - 1, two_streams=1) == B.HA_ERR_WORKSPACE_TOO_SMALL


def step(lib, **kw):
    args = dict(key=FAKE, value=FAKE, sm=FAKE, q=FAKE, kc=FAKE, vc=FAKE, cu=FAKE, sk=FAKE, bt=FAKE,
                out=FAKE, B=3, T=1810, mq=1808, mk=10000, H=2, Hkv=2, D=64, P=16, NB=644, MB=625,
                scale=0.125, dt=B.HA_DTYPE_F32, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.hybrid_step_fwd(*args.values())


def test_step_argument_errors(lib):
    assert step(lib, key=None) == B.HA_ERR_INVALID_ARGUMENT
    assert step(lib, value=None) == B.HA_ERR_INVALID_ARGUMENT
    assert step(lib, sm=None) == B.HA_ERR_INVALID_ARGUMENT
    assert step(lib, Hkv=3) == B.HA_ERR_INVALID_ARGUMENT
    assert step(lib, q=None) == B.HA_ERR_INVALID_ARGUMENT
    assert step(lib, ws=ctypes.c_void_p(0x100010)) == B.HA_ERR_INVALID_ARGUMENT
    assert step(lib, D=96) == B.HA_ERR_UNSUPPORTED
    need = B.workspace_size(3, 1810, 10000, 2, 64)
    assert step(lib, wsb=need - 1) == B.HA_ERR_WORKSPACE_TOO_SMALL
    # no new tokens: nothing to append or attend, nothing enqueued
    assert step(lib, T=0, key=None, value=None, sm=None, wsb=need) == B.HA_OK


def varlen(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, cuk=FAKE, out=FAKE, B=3, T=1810, TK=10167,
                mq=1808, mk=10000, H=2, Hkv=2, D=64, scale=0.125, dt=B.HA_DTYPE_F32, ws=FAKE,
                wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.varlen_attn_fwd(*args.values())


def test_varlen_argument_errors(lib):
    assert varlen(lib, cuk=None) == B.HA_ERR_INVALID_ARGUMENT
    assert varlen(lib, TK=-1) == B.HA_ERR_INVALID_ARGUMENT
    assert varlen(lib, k=None) == B.HA_ERR_INVALID_ARGUMENT
    assert varlen(lib, Hkv=3) == B.HA_ERR_INVALID_ARGUMENT
    assert varlen(lib, mq=20000) == B.HA_ERR_INVALID_ARGUMENT
    assert varlen(lib, D=96) == B.HA_ERR_UNSUPPORTED
    need = B.workspace_size(3, 1810, 10000, 2, 64)
    assert varlen(lib, wsb=need - 1) == B.HA_ERR_WORKSPACE_TOO_SMALL
    assert varlen(lib, T=0, wsb=need) == B.HA_OK


def app(lib, **kw):
    args = dict(key=FAKE, value=FAKE, sm=FAKE, kc=FAKE, vc=FAKE, T=4, Hkv=2, D=128, P=16, NB=8,
                dt=B.HA_DTYPE_BF16, stream=None)
    args.update(kw)
    return lib.paged_kv_append(*args.values())


def test_append_argument_errors(lib):
    assert app(lib, T=-1) == B.HA_ERR_INVALID_ARGUMENT
    assert app(lib, key=None) == B.HA_ERR_INVALID_ARGUMENT
    assert app(lib, kc=None) == B.HA_ERR_INVALID_ARGUMENT
    assert app(lib, NB=0) == B.HA_ERR_INVALID_ARGUMENT
    assert app(lib, D=80) == B.HA_ERR_UNSUPPORTED
    assert app(lib, P=8) == B.HA_ERR_UNSUPPORTED
    assert app(lib, T=0) == B.HA_OK


def test_noalloc_step_argument_errors(lib):
    """hybrid_step_fwd_noalloc rejects bad arguments, and steps whose plan
    arrays alone exceed its 64 MiB scratch array, before touching the GPU."""
    def call(**kw):
        args = dict(key=FAKE, value=FAKE, slot=FAKE, q=FAKE, kc=FAKE, vc=FAKE, cu=FAKE, sk=FAKE,
                    bt=FAKE, out=FAKE, B=3, T=1810, mq=1808, mk=10000, H=2, Hkv=2, D=64, P=16,
                    NB=644, MB=625, scale=0.0, dt=B.HA_DTYPE_F32)
        args.update(kw)
        return lib.hybrid_step_fwd_noalloc(*args.values(), None)
    assert call(key=None) == B.HA_ERR_INVALID_ARGUMENT
    assert call(Hkv=3) == B.HA_ERR_INVALID_ARGUMENT
    assert call(D=96) == B.HA_ERR_UNSUPPORTED
    assert call(bt=None) == B.HA_ERR_INVALID_ARGUMENT
    # 5 million segments: four int32 plan arrays of 20 MB each do not fit
    assert call(B=5_000_000, T=5_000_000, mq=1, mk=16) == B.HA_ERR_WORKSPACE_TOO_SMALL
