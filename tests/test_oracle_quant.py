"""Pins of the oracle's INT2 quantizer and write path: hand-derived group
quantizations and page bytes (tests/golden/), closed-form bounds, exact
round-trips and the region / placement rule of the Italian page ("Architettura
del Sistema di Serving e Layout di Memoria")."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from golden_io import kv_write_spikes, quantizer_groups

GROUPS = quantizer_groups()


@pytest.mark.parametrize("case", GROUPS, ids=[c["name"] for c in GROUPS])
def test_quantizer_golden(case):
    rng = np.random.default_rng(0)
    vals = np.array(case["values"])
    perm = rng.permutation(64)               # order inside the group is irrelevant
    w = np.concatenate([vals[perm], np.zeros(64)])
    codes, s16, z16, *_ = O.quantize(w[None])
    assert int(s16[0, 0].view(np.uint16)) == case["s16"]
    assert int(z16[0, 0].view(np.uint16)) == case["z16"]
    for v, c in case["codes"].items():
        got = codes[0, :64][vals[perm] == v]
        assert (got == c).all(), (v, got, c)


@pytest.mark.parametrize("case", kv_write_spikes(), ids=lambda c: f"{c['kind']}{c['k']}")
def test_kv_write_golden_spikes(case):
    shape = O.Shape(num_kv_heads=1, num_q_heads=1, sink=16, recent=16)
    cache = O.new_cache(shape, num_pages=4, num_slots=1)
    eye = np.zeros((1, 128, 128), np.uint16)
    eye[0, np.arange(128), np.arange(128)] = 0x3F80
    layer = O.Layer(eye, eye, np.float32(case["clip"]), np.float32(case["clip"]))
    sign = np.array([(-1) ** bin(case["k"] & i).count("1") for i in range(128)], np.float64)
    x = O.f64_to_bf16(sign)[None, None]                     # [1][1][128]
    pos = 16 + case["slot"]                                 # page 1, INT2 region
    table = np.array([[0, 1, 2, 3]], np.int32)
    k, v = (x, None) if case["kind"] == "K" else (None, x)
    O.kv_write(shape, cache, layer, k, v, [0], [pos], table, [64])
    blk = cache.pages[1, 0]
    if case["kind"] == "K":
        codes = blk[0:512].copy()
        assert codes[case["index"]] == case["value"]
        codes[case["index"]] = 0
        assert codes.sum() == 0
        par = blk[1024 + 8 * case["slot"]:1024 + 8 * case["slot"] + 8].view("<u2")
    else:
        words = blk[512:1024].copy().view("<u4")
        assert words[case["index"]] == case["value"]
        words[case["index"]] = 0
        assert words.sum() == 0
        par = blk[1152 + 8 * case["slot"]:1152 + 8 * case["slot"] + 8].view("<u2")
    assert list(par) == case["params"]
    # nothing in the ring (pos < L_after - recent) and nothing in the sink
    assert cache.k_ring.sum() == 0 and cache.v_ring.sum() == 0
    assert cache.k_sink.sum() == 0 and cache.v_sink.sum() == 0


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.floats(0.01, 100.0))
def test_quantizer_bounds(seed, spread):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((4, 128)) * spread
    codes, s16, z16, s_pre, z_pre, t = O.quantize(w)
    assert codes.max() <= 3
    s = s16.astype(np.float64)
    z = z16.astype(np.float64)
    g = np.arange(128) // 64
    rec = z[:, g] + s[:, g] * codes
    # half a step plus the fp16 rounding of s (x3 at the top code) and of z
    bound = s[:, g] / 2 + np.abs(z - z_pre)[:, g] + 3 * np.abs(s - s_pre)[:, g] + 1e-12
    assert (np.abs(w - rec) <= bound).all()
    # the group min always decodes to code 0, the group max to code 3
    for r in range(4):
        for gg in range(2):
            seg = w[r, 64 * gg:64 * gg + 64]
            cs = codes[r, 64 * gg:64 * gg + 64]
            assert cs[np.argmin(seg)] == 0 and cs[np.argmax(seg)] == 3


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2 ** 31 - 1))
def test_quantizer_exact_on_grid(seed):
    """Values already on the grid z + s*{0..3} with fp16-exact s, z and both
    ends present round-trip exactly."""
    rng = np.random.default_rng(seed)
    s = float(np.float16(rng.uniform(0.01, 4)))
    z = float(np.float16(rng.uniform(-8, 8)))
    # s must survive (3s)/3 -> fp16 exactly: pick s with a short significand
    s = float(np.float16(np.round(s * 16) / 16))
    if s == 0:
        s = 0.0625
    c = rng.integers(0, 4, 128)
    c[[0, 64]] = 0
    c[[1, 65]] = 3
    w = z + s * c
    codes, s16, z16, *_ = O.quantize(w[None])
    assert float(s16[0, 0]) == s and float(z16[0, 0]) == z
    assert np.array_equal(codes[0], c)


def test_zero_scale_group_gives_zero_codes():
    w = np.full((1, 128), 1.5)
    codes, s16, z16, *_ = O.quantize(w)
    assert codes.sum() == 0 and (s16 == 0).all() and (z16 == 1.5).all()


def test_regions_pins():
    # 64 + 704 + 256 = 1024 (Italian page layout section; tiny workload)
    assert O.regions(1024, 64, 256) == ((0, 64), (64, 768), (768, 1024))
    assert O.regions(320, 64, 256) == ((0, 64), (64, 64), (64, 320))
    assert O.regions(321, 64, 256) == ((0, 64), (64, 65), (65, 321))
    assert O.regions(50, 64, 256) == ((0, 50), (50, 50), (50, 50))
    assert O.regions(1, 64, 256) == ((0, 1), (1, 1), (1, 1))
    assert O.regions(0, 64, 256) == ((0, 0), (0, 0), (0, 0))


def test_write_placement_rule():
    """pos < 64 -> sink row pos; pos >= max(64, L_after-256) -> ring row pos%256;
    pos >= 64 -> INT2 page table[pos//16], slot pos%16."""
    shape = O.Shape(num_kv_heads=2, num_q_heads=2)
    cache = O.new_cache(shape, num_pages=80, num_slots=2)
    rng = np.random.default_rng(5)
    U = np.stack([O.f64_to_bf16(np.linalg.qr(rng.standard_normal((128, 128)))[0]) for _ in range(2)])
    layer = O.Layer(U, U, np.float32(4.0), np.float32(4.0))
    L = 1000
    table = np.zeros((2, 64), np.int32)
    table[0] = rng.permutation(80)[:64]
    pos = np.arange(L)
    x = rng.integers(0x3000, 0x4000, (L, 2, 128)).astype(np.uint16)
    info = O.kv_write(shape, cache, layer, x, x, np.zeros(L, int), pos, table, [L, 0])
    assert np.array_equal(cache.k_sink[0, :, :64], x[:64].transpose(1, 0, 2))
    rows = np.arange(1000 - 256, 1000)
    assert np.array_equal(cache.k_ring[0][:, rows % 256], x[rows].transpose(1, 0, 2))
    assert info["K"]["token"][0] == 64 and len(info["K"]["token"]) == L - 64
    assert np.array_equal(info["K"]["page"], table[0][np.arange(64, L) // 16])
    assert np.array_equal(info["K"]["slot"], np.arange(64, L) % 16)
    # K codes of token 100 are where the format says
    p, sl = table[0][100 // 16], 100 % 16
    got = cache.pages[p, 1, 32 * sl:32 * sl + 32]
    assert np.array_equal(got, O.pack_k_codes(info["K"]["codes"][100 - 64, 1]))
    words = cache.pages[p, 1, 512:1024].copy().view("<u4")
    assert np.array_equal((words >> (2 * sl)) & 3, info["V"]["codes"][100 - 64, 1])
