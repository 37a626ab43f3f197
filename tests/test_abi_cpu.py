"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import exact_io_aware_fwd_amd as xa
from exact_io_aware_fwd_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "exact_attn.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_eight_entry_points():
    assert declared_functions() == ["attn_bwd", "attn_bwd_workspace_size", "attn_fwd", "attn_paged_decode",
                                    "attn_paged_decode_noalloc", "attn_paged_decode_workspace_size",
                                    "attn_paged_prefill", "attn_status_string"]


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    assert xa.status_string(0) == "ok"
    assert "invalid" in xa.status_string(1)
    assert "unsupported" in xa.status_string(2)
    assert "workspace" in xa.status_string(3)
    assert xa.status_string(99) == "unknown status"


def fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=128, scale=0.1,
        kind=0, window=0, doc=None, num_docs=0, dtype=1, sink_tokens=0, sinks=None, softcap=0.0, alibi=None,
        soft=0):
    m = _lib.AttnMask(kind, window, doc, num_docs, sink_tokens, sinks, softcap, alibi, soft)
    return _lib.lib().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, m, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), 2), (dict(d=256), 2), (dict(d=-1), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(Hkv=0), 1), (dict(B=-1), 1), (dict(Nq=-3), 1),
    (dict(dtype=7), 1), (dict(kind=9), 1),
    (dict(kind=2, window=0), 1), (dict(kind=3, num_docs=0, doc=FAKE), 1), (dict(kind=3, num_docs=2, doc=None), 1),
    (dict(scale=0.0), 1), (dict(scale=-1.0), 1), (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1),
    (dict(q=None), 1), (dict(o=None), 1), (dict(k=None), 1), (dict(q=FAKE + 4), 1), (dict(v=FAKE + 8), 1),
    (dict(Nq=1 << 29), 2),
    (dict(kind=1, sink_tokens=4), 1), (dict(kind=0, sink_tokens=1), 1), (dict(kind=2, window=8, sink_tokens=-1), 1),
    (dict(sinks=FAKE + 2), 1), (dict(kind=2, window=8, sink_tokens=4, d=96), 2),
    (dict(softcap=-1.0), 1), (dict(softcap=float("nan")), 1), (dict(softcap=float("inf")), 1),
    (dict(alibi=FAKE + 2), 1), (dict(softcap=-1.0, dtype=0), 1), (dict(softcap=5.0, d=96), 2),
    # the software 2^x: 0, 2 or 4; only bf16, d = 128, no score modifications
    (dict(soft=1), 1), (dict(soft=3), 1), (dict(soft=8), 1), (dict(soft=-2), 1), (dict(soft=3, d=64), 1),
    (dict(soft=2, d=64), 2), (dict(soft=4, dtype=0), 2), (dict(soft=2, softcap=5.0), 2),
    (dict(soft=4, alibi=FAKE), 2), (dict(soft=2, d=96), 2),
])
def test_fwd_rejects_bad_arguments(kw, status):
    assert fwd(**kw) == status


def test_fwd_empty_problems_are_noops():
    # nothing is enqueued, so null pointers are fine
    assert fwd(q=None, k=None, v=None, o=None, lse=None, Nq=0) == 0
    assert fwd(q=None, k=None, v=None, o=None, lse=None, B=0) == 0
    assert fwd(q=None, k=None, v=None, o=None, lse=None, Hq=0, Hkv=0) == 0
    assert fwd(q=None, k=None, v=None, o=None, lse=None, Nq=0, soft=4) == 0


def dec(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=FAKE, S=2, Hq=8, Hkv=2, d=128, page=16,
        max_pages=4, max_len=64, scale=0.1, ws=FAKE, ws_bytes=None, sinks=None, softcap=0.0, alibi=None):
    if ws_bytes is None:
        ws_bytes = xa.attn_paged_decode_workspace_size(S, Hq, d, max_len)
    return _lib.lib().attn_paged_decode(q, kp, vp, bt, sl, o, lse, S, Hq, Hkv, d, page, max_pages, max_len,
                                        scale, sinks, softcap, alibi, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(page=32), 2), (dict(d=96), 2), (dict(Hq=6, Hkv=4), 1), (dict(max_pages=3), 1),
    (dict(S=-1), 1), (dict(scale=0.0), 1), (dict(q=None), 1), (dict(sl=None), 1), (dict(bt=None), 1),
    (dict(kp=FAKE + 2), 1), (dict(ws_bytes=16), 3), (dict(ws=None), 3), (dict(sinks=FAKE + 1), 1),
    (dict(softcap=-1.0), 1), (dict(softcap=float("nan")), 1), (dict(softcap=float("inf")), 1),
    (dict(alibi=FAKE + 2), 1),
])
def test_decode_rejects_bad_arguments(kw, status):
    assert dec(**kw) == status


def test_decode_empty_is_noop():
    assert dec(q=None, o=None, S=0) == 0


def dec_noalloc(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=FAKE, S=2, Hq=8, Hkv=2, d=128, page=16,
                max_pages=4, max_len=64, scale=0.1, sinks=None, softcap=0.0, alibi=None):
    return _lib.lib().attn_paged_decode_noalloc(q, kp, vp, bt, sl, o, lse, S, Hq, Hkv, d, page, max_pages, max_len,
                                                scale, sinks, softcap, alibi, None)


@pytest.mark.parametrize("kw,status", [
    (dict(page=32), 2), (dict(d=96), 2), (dict(Hq=6, Hkv=4), 1), (dict(max_pages=3), 1),
    (dict(S=-1), 1), (dict(scale=0.0), 1), (dict(q=None), 1), (dict(sl=None), 1), (dict(bt=None), 1),
    (dict(kp=FAKE + 2), 1), (dict(sinks=FAKE + 1), 1), (dict(softcap=-1.0), 1), (dict(alibi=FAKE + 2), 1),
    # beyond the scratch array: 64 sequences x 32 heads x 64 1024-key splits x 129 floats > 64 MiB
    (dict(S=64, Hq=32, Hkv=8, max_pages=4096, max_len=65536), 3),
])
def test_decode_noalloc_rejects_bad_arguments_before_any_hip_call(kw, status):
    assert dec_noalloc(**kw) == status


def test_decode_noalloc_limit_is_the_header_constant():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m is not None
    limit = int(m.group(1)) << int(m.group(2))
    f = xa.attn_paged_decode_workspace_size
    assert f(64, 32, 128, 32768) <= limit < f(64, 32, 128, 65536)    # the decode workload fits, twice its length not
    assert dec_noalloc(q=None, o=None, S=0) == 0


def test_workspace_size():
    # one fp32 partial row (d values) and one fp32 LSE per (sequence, query
    # head, 1024-key split), the partial rows rounded up to 256 bytes
    f = xa.attn_paged_decode_workspace_size
    splits = 32768 // 1024
    assert f(64, 32, 128, 32768) >= 64 * 32 * splits * 129 * 4
    assert f(64, 32, 128, 32768) < 64 * 32 * splits * 129 * 4 + 4096
    assert f(64, 32, 128, 1024) < f(64, 32, 128, 1025) <= f(64, 32, 128, 2048)
    assert f(1, 1, 96, 10) == 0 and f(-1, 1, 128, 10) == 0


def chunked(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, qo=FAKE, o=FAKE, lse=FAKE, S=2, Hq=8, Hkv=2, d=128,
            page=16, max_pages=4, max_len=64, max_q=32, scale=0.1, kind=1, window=0, sink_tokens=0, sinks=None,
            softcap=0.0, alibi=None):
    m = _lib.AttnMask(kind, window, None, 0, sink_tokens, sinks, softcap, alibi)
    return _lib.lib().attn_paged_prefill(q, kp, vp, bt, sl, qo, o, lse, S, Hq, Hkv, d, page, max_pages, max_len,
                                         max_q, scale, m, None)


@pytest.mark.parametrize("kw,status", [
    (dict(page=32), 2), (dict(d=96), 2), (dict(kind=3), 2), (dict(kind=7), 1), (dict(kind=2, window=0), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(max_pages=3), 1), (dict(S=-1), 1), (dict(max_q=-1), 1),
    (dict(scale=0.0), 1), (dict(scale=float("nan")), 1), (dict(q=None), 1), (dict(qo=None), 1),
    (dict(sl=None), 1), (dict(bt=None), 1), (dict(kp=FAKE + 2), 1), (dict(o=FAKE + 8), 1),
    (dict(max_len=1 << 29, max_pages=1 << 25), 2),
    (dict(kind=1, sink_tokens=2), 1), (dict(sinks=FAKE + 2), 1),
    (dict(softcap=-2.0), 1), (dict(softcap=float("nan")), 1), (dict(alibi=FAKE + 1), 1),
])
def test_paged_prefill_rejects_bad_arguments(kw, status):
    assert chunked(**kw) == status


def test_paged_prefill_empty_problems_are_noops():
    assert chunked(q=None, kp=None, vp=None, bt=None, sl=None, qo=None, o=None, lse=None, S=0) == 0
    assert chunked(q=None, kp=None, vp=None, bt=None, sl=None, qo=None, o=None, lse=None, max_q=0) == 0


def bwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, dsink=None, B=1, Hq=4, Hkv=2,
        Nq=16, Nk=16, d=128, scale=0.1, kind=1, window=0, dtype=1, ws=FAKE, ws_bytes=None, sink_tokens=0, sinks=None,
        softcap=0.0, alibi=None):
    if ws_bytes is None:
        ws_bytes = xa.attn_bwd_workspace_size(B, Hq, Nq)
    m = _lib.AttnMask(kind, window, None, 0, sink_tokens, sinks, softcap, alibi)
    return _lib.lib().attn_bwd(q, k, v, o, do, lse, dq, dk, dv, dsink, B, Hq, Hkv, Nq, Nk, d, scale, m, dtype,
                               ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), 2), (dict(d=96, dtype=0), 2), (dict(dtype=5), 1), (dict(Hq=6, Hkv=4), 1), (dict(B=-1), 1),
    (dict(scale=0.0), 1), (dict(kind=9), 1), (dict(kind=2, window=0), 1), (dict(kind=1, sink_tokens=3), 1),
    (dict(q=None), 1), (dict(do=None), 1), (dict(lse=None), 1), (dict(dk=None), 1), (dict(dq=FAKE + 8), 1),
    (dict(lse=FAKE + 2), 1), (dict(ws_bytes=8), 3), (dict(ws=None), 3), (dict(Nk=1 << 29), 2),
    (dict(softcap=-5.0), 1), (dict(softcap=float("nan")), 1), (dict(alibi=FAKE + 2), 1),
    (dict(softcap=5.0, d=96), 2),
])
def test_bwd_rejects_bad_arguments(kw, status):
    assert bwd(**kw) == status


def test_bwd_workspace_size():
    assert xa.attn_bwd_workspace_size(2, 4, 100) == 4 * (((2 * 4 * 100 * 4) + 255) // 256) * 256
    assert xa.attn_bwd_workspace_size(-1, 4, 100) == 0
    assert bwd(q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None, B=0) == 0


def test_binding_fails_loudly_without_the_library(monkeypatch):
    # no fallback: with the shared library absent the binding raises
    monkeypatch.setattr(_lib, "LIB_PATH", _lib.LIB_PATH + ".absent")
    monkeypatch.setattr(_lib, "_lib", None)          # the cached handle
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()
    with pytest.raises(RuntimeError, match="missing"):
        xa.status_string(0)
