"""C ABI checks that need no GPU: the library loads, exports every declared entry point, and
rejects invalid arguments on the host before any HIP call.

Fake device pointers below are only ever passed together with an argument the host check
rejects, so no kernel is launched and nothing is dereferenced.
"""
import ctypes
import os
import re

import pytest

from oracle import group_size
from zero_shot_rope_amd import bifocal as B
from zero_shot_rope_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bifocal.h")
OK, EINVAL, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4
FAKE = 0x1000  # never dereferenced: every call using it fails a host-side check first


def odd_float_ptr(offset):
    """A float* argument FAKE + offset (not 4-byte aligned for odd offsets below 4)."""
    return ctypes.cast(ctypes.c_void_p(FAKE + offset), ctypes.POINTER(ctypes.c_float))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build_mod.LIB):
        build_mod.build()
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bifocal_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(B.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(B.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_group_size_matches_oracle(lib):
    for L in list(range(1, 300)) + [32767, 32768, 32769, 65536, 98304, 98305, 131072, 1 << 30]:
        for wp in (1, 7, 128, 32768):
            assert B.bifocal_group_size(L, wp) == group_size(L, wp)


def test_group_size_rejects_bad_arguments(lib):
    for L, wp in [(0, 1), (-1, 5), (5, 0), (5, -2)]:
        assert lib.bifocal_group_size(L, wp) == EINVAL


def test_status_strings(lib):
    seen = set()
    for st in (OK, EINVAL, EUNSUP, EWS, EHIP):
        s = B.bifocal_status_string(st)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 5
    assert B.bifocal_status_string(12345) == "unknown status"


def prefill_call(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, batch=1, hq=4, hkv=2, d=128, L=256, w0=32,
                wp=64, theta=1e4)
    args.update(kw)
    args.setdefault("ws", None)
    args.setdefault("wsb", 0)
    return lib.bifocal_prefill(args["q"], args["k"], args["v"], args["o"], args["lse"], args["batch"],
                               args["hq"], args["hkv"], args["d"], args["L"], args["w0"], args["wp"],
                               args["theta"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), EINVAL), (dict(k=None), EINVAL), (dict(v=None), EINVAL), (dict(o=None), EINVAL),
    (dict(batch=0), EINVAL), (dict(hq=0), EINVAL), (dict(hkv=0), EINVAL), (dict(d=0), EINVAL),
    (dict(L=0), EINVAL), (dict(L=-5), EINVAL), (dict(w0=-1), EINVAL), (dict(wp=0), EINVAL),
    (dict(theta=0.0), EINVAL), (dict(theta=-1.0), EINVAL), (dict(theta=float("nan")), EINVAL),
    (dict(theta=float("inf")), EINVAL), (dict(hq=6, hkv=4), EINVAL),
    (dict(d=96), EUNSUP), (dict(d=256), EUNSUP), (dict(L=(1 << 30) + 1), EUNSUP),
    (dict(hq=1 << 17, hkv=1 << 17), EUNSUP),  # n_kv_heads * head_dim = 2^24: 32-bit tile offsets
    (dict(ws=FAKE, wsb=0), EWS), (dict(ws=FAKE, wsb=256 * 2 * 128 * 2 - 1), EWS),
    (dict(q=FAKE + 2), EINVAL), (dict(k=FAKE + 8), EINVAL), (dict(v=FAKE + 4), EINVAL), (dict(o=FAKE + 2), EINVAL),
    (dict(lse=odd_float_ptr(2)), EINVAL), (dict(ws=FAKE + 8, wsb=1 << 40), EINVAL),
])
def test_prefill_rejects_before_any_hip_call(lib, kw, expect):
    assert prefill_call(lib, **kw) == expect


def chunk_call(lib, **kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, batch=1, hq=4, hkv=2, d=128, q_len=100, q_off=50, cap=200,
                w0=32, wp=64, theta=1e4, ws=None, wsb=0)
    args.update(kw)
    return lib.bifocal_prefill_chunk(args["q"], args["kc"], args["vc"], args["o"], args["lse"], args["batch"], args["hq"],
                                     args["hkv"], args["d"], args["q_len"], args["q_off"], args["cap"], args["w0"],
                                     args["wp"], args["theta"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), EINVAL), (dict(kc=None), EINVAL), (dict(vc=None), EINVAL), (dict(o=None), EINVAL),
    (dict(q_len=0), EINVAL), (dict(q_off=-1), EINVAL), (dict(q_off=101), EINVAL), (dict(q_len=201, q_off=0), EINVAL),
    (dict(cap=0), EINVAL), (dict(w0=-1), EINVAL), (dict(wp=0), EINVAL), (dict(theta=0.0), EINVAL),
    (dict(hq=6, hkv=4), EINVAL), (dict(batch=0), EINVAL), (dict(d=96), EUNSUP),
    (dict(cap=(1 << 30) + 1, q_off=0), EUNSUP),
    (dict(ws=FAKE, wsb=150 * 2 * 128 * 2 - 1), EWS),   # sized for L = q_off + q_len = 150
    (dict(kc=FAKE + 2), EINVAL), (dict(vc=FAKE + 8), EINVAL), (dict(lse=odd_float_ptr(1)), EINVAL),
])
def test_prefill_chunk_rejects_before_any_hip_call(lib, kw, expect):
    assert chunk_call(lib, **kw) == expect


def decode_call(lib, **kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, batch=1, hq=8, hkv=2, d=128, L=100, cap=128,
                w0=16, wp=32, theta=1e4, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    return lib.bifocal_decode(args["q"], args["kc"], args["vc"], args["o"], args["lse"], args["batch"], args["hq"],
                              args["hkv"], args["d"], args["L"], args["cap"], args["w0"], args["wp"], args["theta"],
                              args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), EINVAL), (dict(kc=None), EINVAL), (dict(vc=None), EINVAL), (dict(o=None), EINVAL),
    (dict(L=0), EINVAL), (dict(L=129), EINVAL), (dict(w0=-3), EINVAL), (dict(wp=0), EINVAL),
    (dict(theta=0.0), EINVAL), (dict(hq=7, hkv=2), EINVAL), (dict(batch=0), EINVAL),
    (dict(d=80), EUNSUP), (dict(hq=34, hkv=2), EUNSUP), (dict(hq=64, hkv=2), EUNSUP),
    (dict(ws=None), EWS), (dict(wsb=0), EWS), (dict(wsb=16), EWS),
    (dict(q=FAKE + 2), EINVAL), (dict(kc=FAKE + 8), EINVAL), (dict(vc=FAKE + 4), EINVAL), (dict(o=FAKE + 2), EINVAL),
    (dict(lse=odd_float_ptr(2)), EINVAL), (dict(ws=FAKE + 8), EINVAL),
])
def test_decode_rejects_before_any_hip_call(lib, kw, expect):
    assert decode_call(lib, **kw) == expect


def step_call(lib, **kw):
    args = dict(qr=FAKE, kr=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, batch=1, hq=8, hkv=2, d=128, L=100,
                cap=128, w0=16, wp=32, theta=1e4, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    return lib.bifocal_decode_step(args["qr"], args["kr"], args["vn"], args["kc"], args["vc"], args["o"], args["lse"],
                                   args["batch"], args["hq"], args["hkv"], args["d"], args["L"], args["cap"],
                                   args["w0"], args["wp"], args["theta"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(qr=None), EINVAL), (dict(kr=None), EINVAL), (dict(vn=None), EINVAL), (dict(kc=None), EINVAL),
    (dict(vc=None), EINVAL), (dict(o=None), EINVAL), (dict(L=0), EINVAL), (dict(L=129), EINVAL),
    (dict(w0=-1), EINVAL), (dict(wp=0), EINVAL), (dict(theta=float("nan")), EINVAL), (dict(hq=6, hkv=4), EINVAL),
    (dict(d=96), EUNSUP), (dict(hq=34, hkv=2), EUNSUP), (dict(cap=(1 << 30) + 1), EUNSUP), (dict(ws=None), EWS),
    (dict(wsb=0), EWS), (dict(qr=FAKE + 2), EINVAL), (dict(kr=FAKE + 2), EINVAL), (dict(vn=FAKE + 8), EINVAL),
    (dict(kc=FAKE + 4), EINVAL),
])
def test_decode_step_rejects_before_any_hip_call(lib, kw, expect):
    # Every rejection happens before the cache row is written (the fake pointers are never touched).
    assert step_call(lib, **kw) == expect


def varlen_call(lib, **kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, batch=3, hq=8, hkv=2, d=128, lens=FAKE, max_len=100,
                cap=128, w0=16, wp=32, theta=1e4, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    return lib.bifocal_decode_varlen(args["q"], args["kc"], args["vc"], args["o"], args["lse"], args["batch"],
                                     args["hq"], args["hkv"], args["d"], args["lens"], args["max_len"], args["cap"],
                                     args["w0"], args["wp"], args["theta"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(lens=None), EINVAL), (dict(q=None), EINVAL), (dict(max_len=0), EINVAL), (dict(max_len=129), EINVAL),
    (dict(w0=-1), EINVAL), (dict(wp=0), EINVAL), (dict(theta=-2.0), EINVAL), (dict(batch=0), EINVAL),
    (dict(d=80), EUNSUP), (dict(hq=34, hkv=2), EUNSUP), (dict(ws=None), EWS), (dict(wsb=16), EWS),
    (dict(lens=ctypes.cast(ctypes.c_void_p(FAKE + 2), ctypes.POINTER(ctypes.c_int32))), EINVAL), (dict(q=FAKE + 8), EINVAL),
])
def test_decode_varlen_rejects_before_any_hip_call(lib, kw, expect):
    assert varlen_call(lib, **kw) == expect


def test_decode_varlen_workspace_query(lib):
    assert lib.bifocal_decode_varlen_workspace_bytes(0, 8, 2, 128, 100) == 0
    # One partial record (all query heads, D + 2 floats each) per segment: at most one grid of
    # workgroups (256 per KV-head group of 8) plus the batch; then a (first, count) int32 pair per
    # sequence. Linear in the batch and independent of the length.
    for B, Hq, Hkv, D in [(3, 32, 8, 128), (4096, 32, 8, 128), (5, 64, 16, 64)]:
        wgs = -(-256 // -(-Hkv // 8))
        want = (wgs + B) * Hq * (D + 2) * 4 + B * 8
        for L in [1, 33, 98001, 131072]:
            assert lib.bifocal_decode_varlen_workspace_bytes(B, Hq, Hkv, D, L) == want
    need = lib.bifocal_decode_varlen_workspace_bytes(3, 8, 2, 128, 100)
    assert varlen_call(lib, wsb=need - 1) == EWS


def test_decode_workspace_query(lib):
    assert lib.bifocal_decode_workspace_bytes(0, 8, 2, 128, 100) == 0
    assert lib.bifocal_decode_workspace_bytes(1, 8, 3, 128, 100) == 0
    prev = 0
    for L in [1, 31, 32, 33, 1000, 4096, 98001, 98512, 131072]:
        n = lib.bifocal_decode_workspace_bytes(1, 32, 8, 128, L)
        assert n >= prev and n % (130 * 4 * 32) == 0
        prev = n
    # The exact requirement is accepted (the call still fails later only on the fake data).
    need = lib.bifocal_decode_workspace_bytes(1, 8, 2, 128, 100)
    assert decode_call(lib, wsb=need - 1) == EWS


def test_positions_rejects_bad_arguments(lib):
    p = ctypes.cast(ctypes.c_void_p(FAKE), ctypes.POINTER(ctypes.c_int32))
    assert lib.bifocal_positions(10, 4, None, p, None) == EINVAL
    assert lib.bifocal_positions(10, 4, p, None, None) == EINVAL
    assert lib.bifocal_positions(0, 4, p, p, None) == EINVAL
    assert lib.bifocal_positions(10, 0, p, p, None) == EINVAL
    assert lib.bifocal_positions(1 << 31, 4, p, p, None) == EINVAL
    odd = ctypes.cast(ctypes.c_void_p(FAKE + 2), ctypes.POINTER(ctypes.c_int32))
    assert lib.bifocal_positions(10, 4, odd, p, None) == EINVAL
    assert lib.bifocal_positions(10, 4, p, odd, None) == EINVAL


def test_binding_refuses_to_run_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("BIFOCAL_LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.load_library()


def test_prefill_workspace_query(lib):
    assert lib.bifocal_prefill_workspace_bytes(1, 8, 128, 131072) == 131072 * 8 * 128 * 2
    assert lib.bifocal_prefill_workspace_bytes(2, 2, 64, 100) == 2 * 100 * 2 * 64 * 2
    for bad in [(0, 8, 128, 10), (1, 0, 128, 10), (1, 8, 96, 10), (1, 8, 128, 0), (1, 8, 128, (1 << 30) + 1)]:
        assert lib.bifocal_prefill_workspace_bytes(*bad) == 0


def prefill_unfused_call(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, batch=1, hq=4, hkv=2, d=128, L=256, w0=32, wp=64,
                theta=1e4, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    return lib.bifocal_prefill_unfused(args["q"], args["k"], args["v"], args["o"], args["lse"], args["batch"],
                                       args["hq"], args["hkv"], args["d"], args["L"], args["w0"], args["wp"],
                                       args["theta"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), EINVAL), (dict(k=None), EINVAL), (dict(v=None), EINVAL), (dict(o=None), EINVAL),
    (dict(batch=0), EINVAL), (dict(L=0), EINVAL), (dict(w0=-1), EINVAL), (dict(wp=0), EINVAL),
    (dict(theta=0.0), EINVAL), (dict(hq=6, hkv=4), EINVAL), (dict(d=96), EUNSUP), (dict(L=(1 << 30) + 1), EUNSUP),
    (dict(ws=None), EWS), (dict(wsb=0), EWS), (dict(q=FAKE + 2), EINVAL), (dict(ws=FAKE + 4), EINVAL),
])
def test_prefill_unfused_rejects_before_any_hip_call(lib, kw, expect):
    assert prefill_unfused_call(lib, **kw) == expect


def test_prefill_unfused_workspace_query(lib):
    assert lib.bifocal_prefill_unfused_workspace_bytes(0, 4, 2, 128, 256) == 0
    assert lib.bifocal_prefill_unfused_workspace_bytes(1, 4, 2, 96, 256) == 0
    # q' + k' + three pass outputs (fp32) + three LSEs (fp32), each region 256-byte aligned.
    B, Hq, Hkv, D, L = 2, 4, 2, 128, 300
    q, k, lse = B * L * Hq * D * 2, B * L * Hkv * D * 2, B * Hq * L * 4
    a = lambda x: (x + 255) // 256 * 256
    assert lib.bifocal_prefill_unfused_workspace_bytes(B, Hq, Hkv, D, L) == a(q) + a(k) + 3 * a(2 * q) + 3 * a(lse)
    need = lib.bifocal_prefill_unfused_workspace_bytes(1, 4, 2, 128, 256)
    assert prefill_unfused_call(lib, wsb=need - 1) == EWS


def decode_unfused_call(lib, **kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, batch=1, hq=8, hkv=2, d=128, L=100, cap=128,
                w0=16, wp=32, theta=1e4, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    return lib.bifocal_decode_unfused(args["q"], args["kc"], args["vc"], args["o"], args["lse"], args["batch"],
                                      args["hq"], args["hkv"], args["d"], args["L"], args["cap"], args["w0"],
                                      args["wp"], args["theta"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), EINVAL), (dict(kc=None), EINVAL), (dict(vc=None), EINVAL), (dict(o=None), EINVAL),
    (dict(L=0), EINVAL), (dict(L=129), EINVAL), (dict(w0=-3), EINVAL), (dict(wp=0), EINVAL),
    (dict(theta=0.0), EINVAL), (dict(hq=7, hkv=2), EINVAL), (dict(batch=0), EINVAL),
    (dict(d=80), EUNSUP), (dict(hq=34, hkv=2), EUNSUP), (dict(cap=(1 << 30) + 1), EUNSUP),
    (dict(ws=None), EWS), (dict(wsb=1024), EWS), (dict(kc=FAKE + 2), EINVAL), (dict(ws=FAKE + 8), EINVAL),
])
def test_decode_unfused_rejects_before_any_hip_call(lib, kw, expect):
    assert decode_unfused_call(lib, **kw) == expect


def test_decode_unfused_workspace_query(lib):
    assert lib.bifocal_decode_unfused_workspace_bytes(0, 8, 2, 128, 128) == 0
    n = lib.bifocal_decode_unfused_workspace_bytes(1, 8, 2, 128, 128)
    # At least the rotated key copy plus the split workspace of a plain decode.
    assert n >= 128 * 2 * 128 * 2 + lib.bifocal_decode_workspace_bytes(1, 8, 2, 128, 128)
    assert decode_unfused_call(lib, wsb=n - 1) == EWS
