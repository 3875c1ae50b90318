"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/oscar.h declares, and rejects bad arguments before
any device work."""
import ctypes
import os
import re

import pytest

import int2_rotated_kv_write_amd as lib
from int2_rotated_kv_write_amd._native import OscarLayer, OscarShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# A stand-in device address: 256-byte aligned, never dereferenced (every call below
# that passes it fails a host-side check, or has nothing to do, before any launch).
A = 0x10000


def header_functions():
    text = open(os.path.join(ROOT, "include", "oscar.h")).read()
    return sorted(set(re.findall(r"\b(oscar_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = lib.load()
    names = header_functions()
    assert len(names) >= 6
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert lib.status_string(0) == "ok"
    assert lib.status_string(1) == "invalid argument"
    assert lib.status_string(2) == "workspace too small"
    assert lib.status_string(3) == "HIP error"


def good_shape(**kw):
    d = dict(num_kv_heads=8, num_q_heads=32, head_dim=128, page_size=16, sink=64, recent=256, group=64)
    d.update(kw)
    return OscarShape(**d)


@pytest.mark.parametrize("bad", [
    dict(head_dim=64), dict(page_size=32), dict(group=32), dict(group=256), dict(num_kv_heads=0),
    dict(num_q_heads=30), dict(num_q_heads=8 * 9), dict(sink=10), dict(sink=2048),
    dict(recent=0), dict(recent=5000),
])
def test_bad_shapes_rejected(bad):
    L = lib.load()
    s = good_shape(**bad)
    layer = OscarLayer()
    rc = L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), 1, 1, 1, 1, 4, 1, 8, 1, None)
    assert rc == 1
    assert L.oscar_decode_workspace_bytes(ctypes.byref(s), 2, 10) == 0
    rc = L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), 1, 1, 8, 1, 2, 0.1, 1, 1, 1 << 30, None)
    assert rc == 1
    assert L.oscar_last_error()


def test_null_and_range_arguments_rejected():
    L = lib.load()
    s = good_shape()
    assert L.oscar_kv_write(None, None, 1, 1, 1, 1, 4, 1, 8, 1, None) == 1
    layer = OscarLayer(pages=A, k_sink=A, v_sink=A, k_ring=A, v_ring=A, u_k=A, u_v=A,
                       clip_k=4.0, clip_v=4.0)
    # negative token count, zero max_pages, NULL index arrays
    assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), 1, 1, 1, 1, -1, 1, 8, 1, None) == 1
    assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), 1, 1, 1, 1, 4, 1, 0, 1, None) == 1
    assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), 1, 1, None, 1, 4, 1, 8, 1, None) == 1
    # clip thresholds must be finite and in (0, 16384]
    for c in (0.0, -1.0, float("inf"), float("nan"), 20000.0):
        bad = OscarLayer(pages=A, k_sink=A, v_sink=A, k_ring=A, v_ring=A, u_k=A, u_v=A, clip_k=c, clip_v=4.0)
        assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(bad), 1, None, 1, 1, 4, 1, 8, 1, None) == 1
    # zero tokens, or neither k nor v: nothing to do
    assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), 1, 1, 1, 1, 0, 1, 8, 1, None) == 0
    assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), None, None, 1, 1, 4, 1, 8, 1, None) == 0


def test_decode_workspace_checks():
    L = lib.load()
    s = good_shape()
    layer = OscarLayer(pages=A, k_sink=A, v_sink=A, k_ring=A, v_ring=A, u_k=A, u_v=A,
                       clip_k=4.0, clip_v=4.0)
    need = L.oscar_decode_workspace_bytes(ctypes.byref(s), 28, 6250)
    assert need > 28 * 32 * 320
    # too small -> ENOWS; misaligned -> EINVAL; batch 0 -> OK without touching anything
    rc = L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), A, A, 6250, A, 28, 0.088, A, 256, need - 1, None)
    assert rc == 2
    rc = L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), A, A, 6250, A, 28, 0.088, A, 257, need, None)
    assert rc == 1
    rc = L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), A, A, 6250, A, 0, 0.088, A, None, 0, None)
    assert rc == 0
    rc = L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), None, A, 6250, A, 28, 0.088, A, 256, need, None)
    assert rc == 1
    rc = L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), A, A, 6250, A, 28, float("nan"), A, 256, need,
                             None)
    assert rc == 1


def test_workspace_grows_with_batch_and_pages():
    L = lib.load()
    s = good_shape()
    a = L.oscar_decode_workspace_bytes(ctypes.byref(s), 1, 100)
    b = L.oscar_decode_workspace_bytes(ctypes.byref(s), 2, 100)
    c = L.oscar_decode_workspace_bytes(ctypes.byref(s), 2, 10000)
    assert 0 < a < b < c


def test_workspace_max_pages_limit():
    """One call splits the INT2 pages after the sink pages into at most 1,023
    ranges of at most 512 pages: max_pages = sink/16 + 523,776 is the largest
    accepted (about 8.4M tokens), one more page is rejected with size 0."""
    L = lib.load()
    s = good_shape()
    top = s.sink // 16 + 1023 * 512
    assert L.oscar_decode_workspace_bytes(ctypes.byref(s), 1, top) > 0
    assert L.oscar_decode_workspace_bytes(ctypes.byref(s), 1, top + 1) == 0


def test_bf16_decode_argument_checks():
    """The BF16 baseline decode: bad head counts, NaN scale, NULL pointers and
    small or misaligned workspaces are rejected on the host; batch 0 is a no-op."""
    L = lib.load()
    need = L.oscar_bf16_decode_workspace_bytes(8, 32, 28, 6250)
    assert need >= 28 * 32 * 16 * (128 * 4 + 8)   # at least 16 ranges per (sequence, KV head) at 100K
    for h, hq in ((0, 8), (8, 30), (1, 9)):
        assert L.oscar_bf16_decode_workspace_bytes(h, hq, 2, 10) == 0
        assert L.oscar_bf16_decode_attn(h, hq, 1, 1, 1, 10, 1, 2, 0.088, 1, 256, 1 << 30, None) == 1
    assert L.oscar_bf16_decode_workspace_bytes(8, 32, 2, 0) == 0
    args = lambda **kw: dict(dict(pages=A, q=A, table=A, mp=6250, lens=A, B=28, sc=0.088, out=A, ws=256, n=need), **kw)
    call = lambda a: L.oscar_bf16_decode_attn(8, 32, a["pages"], a["q"], a["table"], a["mp"], a["lens"], a["B"],
                                              a["sc"], a["out"], a["ws"], a["n"], None)
    assert call(args(n=need - 1)) == 2
    assert call(args(ws=257)) == 1
    assert call(args(pages=None)) == 1
    assert call(args(sc=float("inf"))) == 1
    assert call(args(mp=0)) == 1
    assert call(args(B=0, ws=None, n=0)) == 0
    assert a_grows(L)


def a_grows(L):
    a = L.oscar_bf16_decode_workspace_bytes(8, 32, 1, 100)
    b = L.oscar_bf16_decode_workspace_bytes(8, 32, 2, 100)
    c = L.oscar_bf16_decode_workspace_bytes(8, 32, 2, 10000)
    return 0 < a < b < c


def test_read_probe_argument_checks():
    L = lib.load()
    need = L.oscar_read_probe_sink_bytes()
    assert need > 0
    assert L.oscar_read_probe(None, 1 << 20, 256, need, None) == 1
    assert L.oscar_read_probe(256, 1 << 20, None, need, None) == 1
    assert L.oscar_read_probe(256, 0, 256, need, None) == 1
    assert L.oscar_read_probe(256, 100, 256, need, None) == 1
    assert L.oscar_read_probe(264, 1 << 20, 256, need, None) == 1
    assert L.oscar_read_probe(256, 1 << 20, 256, need - 1, None) == 2


def test_decode_step_checks_both_halves_before_launching():
    """decode_step = kv_write then decode_attn: a bad argument of either half is
    rejected on the host (nothing launched); empty halves are no-ops."""
    L = lib.load()
    s = good_shape()
    layer = OscarLayer(pages=A, k_sink=A, v_sink=A, k_ring=A, v_ring=A, u_k=A, u_v=A, clip_k=4.0, clip_v=4.0)
    need = L.oscar_decode_workspace_bytes(ctypes.byref(s), 28, 6250)

    def step(**kw):
        a = dict(k=A, v=A, idx=A, pos=A, T=28, after=A, q=A, table=A, mp=6250, lens=A, B=28, sc=0.088, out=A,
                 ws=256, n=need, shape=s, layer=layer)
        a.update(kw)
        return L.oscar_decode_step(ctypes.byref(a["shape"]), ctypes.byref(a["layer"]), a["k"], a["v"], a["idx"],
                                   a["pos"], a["T"], a["after"], a["q"], a["table"], a["mp"], a["lens"], a["B"],
                                   a["sc"], a["out"], a["ws"], a["n"], None)

    assert step(shape=good_shape(head_dim=64)) == 1
    assert step(T=-1) == 1                     # write half
    assert step(idx=None) == 1
    assert step(layer=OscarLayer(pages=A, k_sink=A, v_sink=A, k_ring=A, v_ring=A, u_k=A, u_v=A,
                                 clip_k=0.0, clip_v=4.0)) == 1
    assert step(sc=float("nan")) == 1          # decode half
    assert step(q=None) == 1
    assert step(n=need - 1) == 2
    assert step(ws=257) == 1
    assert step(T=0, B=0) == 0                 # both halves empty
    assert step(k=None, v=None, B=0) == 0


def test_misaligned_pointers_rejected():
    """16-byte alignment of bf16 / byte tensors and 4-byte alignment of int32
    arrays are checked on the host before any launch."""
    L = lib.load()
    s = good_shape()
    good = dict(pages=A, k_sink=A, v_sink=A, k_ring=A, v_ring=A, u_k=A, u_v=A, clip_k=4.0, clip_v=4.0)
    need = L.oscar_decode_workspace_bytes(ctypes.byref(s), 28, 6250)
    for f in ("pages", "k_sink", "v_sink", "k_ring", "v_ring", "u_k", "u_v"):
        layer = OscarLayer(**dict(good, **{f: A + 8}))
        assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), A, A, A, A, 4, A, 8, A, None) == 1
        assert b"16-byte" in L.oscar_last_error()
        assert L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), A, A, 6250, A, 28, 0.088, A, 256, need,
                                   None) == 1
    layer = OscarLayer(**good)
    for k, v in ((A + 2, A), (A, A + 4)):
        assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), k, v, A, A, 4, A, 8, A, None) == 1
    for idx, pos, table, after in ((A + 2, A, A, A), (A, A + 1, A, A), (A, A, A + 2, A), (A, A, A, A + 3)):
        assert L.oscar_kv_write(ctypes.byref(s), ctypes.byref(layer), A, A, idx, pos, 4, table, 8, after, None) == 1
        assert b"4-byte" in L.oscar_last_error()
    for q, table, lens, out in ((A + 8, A, A, A), (A, A + 2, A, A), (A, A, A + 2, A), (A, A, A, A + 2)):
        assert L.oscar_decode_attn(ctypes.byref(s), ctypes.byref(layer), q, table, 6250, lens, 28, 0.088, out, 256,
                                   need, None) == 1
    assert L.oscar_bf16_decode_attn(8, 32, A + 8, A, A, 6250, A, 28, 0.088, A, 256, 1 << 40, None) == 1


def test_noalloc_decode_host_checks():
    """decode_attn_noalloc: argument errors and a call whose scratch need exceeds
    the static array are rejected on the host (nothing looked up or launched);
    batch 0 is a no-op."""
    L = lib.load()
    s = good_shape()
    layer = OscarLayer(pages=A, k_sink=A, v_sink=A, k_ring=A, v_ring=A, u_k=A, u_v=A, clip_k=4.0, clip_v=4.0)
    call = lambda **kw: L.oscar_decode_attn_noalloc(
        ctypes.byref(kw.get("shape", s)), ctypes.byref(layer), kw.get("q", A), A, kw.get("mp", 6250), A,
        kw.get("B", 28), kw.get("sc", 0.088), A, None)
    assert call(shape=good_shape(head_dim=64)) == 1
    assert call(B=-1) == 1
    assert call(mp=0) == 1
    assert call(B=0) == 0
    top = s.sink // 16 + 1023 * 512
    assert L.oscar_decode_workspace_bytes(ctypes.byref(s), 64, top) > (64 << 20)
    assert call(B=64, mp=top) == 1
    assert b"OSCAR_NOALLOC_SCRATCH_BYTES" in L.oscar_last_error()
    assert call(B=1, mp=top + 1) == 1            # beyond what one call can split at all
