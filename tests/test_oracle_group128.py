"""Pins of the oracle's 128-channel-group format (one fp16 scale and zero per
token and head: 2.25 bits per element, the format behind the Russian page's
paragraph 4 figure of "2.28 bits per KV element"), each against something
other than the function itself: the block size that 2.25 bits gives, exact
round trips on an fp16 grid, the reduction to the 64-channel quantizer when
both halves share one range, the hand-derived spike bytes of
tests/golden/kv_write_spikes.txt (a single non-zero rotated channel gives the
same codes and the spike group's (s, z) whatever the grouping), and the
reconstruction bound of the min/max quantizer through kv_write and decode."""
import math

import numpy as np
import pytest

import oracle as O
import synth
from golden_io import kv_write_spikes
from test_oracle_attention import brute_attention, random_layer

SIG = 1 / math.sqrt(128)


def test_block_sizes_are_the_bits_per_element():
    """16 tokens x (K + V) x 128 channels: 2 bits of code plus 32 bits of fp16 (s, z)
    per group, i.e. 2.5 bits per element with 64-channel groups and 2.25 with 128."""
    for group, bits in ((64, 2.5), (128, 2.25)):
        blk, k_par, v_par, pb = O.block_layout(group)
        assert blk == 16 * 2 * 128 * bits / 8
        assert pb == 4 * (128 // group)
        assert k_par == 1024 and v_par == k_par + 16 * pb and blk == v_par + 16 * pb
    with pytest.raises(ValueError):
        O.block_layout(32)


def test_exact_on_an_fp16_grid():
    """w = z + s code with fp16 s, z and a 0 and a 3 in every row: the quantizer
    returns exactly those codes, s and z (one group over all 128 channels)."""
    rng = np.random.default_rng(1)
    n = 200
    s = O.fp16_rne(rng.uniform(0.01, 2.0, n)).astype(np.float64)
    z = O.fp16_rne(rng.uniform(-3.0, 1.0, n)).astype(np.float64)
    codes = rng.integers(0, 4, (n, 128))
    codes[:, 3], codes[:, 77] = 0, 3
    w = z[:, None] + s[:, None] * codes
    got, s16, z16, *_ = O.quantize(w, 128)
    assert s16.shape == (n, 1)
    assert np.array_equal(got, codes)
    assert np.array_equal(s16[:, 0].astype(np.float64), s)
    assert np.array_equal(z16[:, 0].astype(np.float64), z)


def test_reduces_to_64_channel_groups_when_the_halves_share_a_range():
    rng = np.random.default_rng(2)
    w = np.clip(rng.standard_normal((50, 128)), -3.5, 2.5)
    for half in (0, 64):                       # plant the same min and max in both halves
        w[:, half + 5] = -4.0
        w[:, half + 9] = 3.0
    c128, s128, z128, *_ = O.quantize(w, 128)
    c64, s64, z64, *_ = O.quantize(w, 64)
    assert np.array_equal(c128, c64)
    for g in range(2):
        assert np.array_equal(s128[:, 0], s64[:, g]) and np.array_equal(z128[:, 0], z64[:, g])


def test_one_range_over_both_halves():
    """Half the channels at 0 and half at 3: s = 1, z = 0, codes 0 and 3 -- while
    64-channel groups see two flat groups (s = 0) with zero points 0 and 3."""
    w = np.concatenate([np.zeros(64), np.full(64, 3.0)])[None]
    c, s, z, *_ = O.quantize(w, 128)
    assert float(s[0, 0]) == 1.0 and float(z[0, 0]) == 0.0
    assert (c[0, :64] == 0).all() and (c[0, 64:] == 3).all()
    c64, s64, z64, *_ = O.quantize(w, 64)
    assert (s64 == 0).all() and list(z64[0]) == [0.0, 3.0] and (c64 == 0).all()


@pytest.mark.parametrize("case", kv_write_spikes(), ids=lambda c: f"{c['kind']}{c['k']}")
def test_spike_bytes(case):
    """The golden spikes: one rotated channel is non-zero, so the token's single
    group has the spike group's (s, z) and the same codes; parameters sit at
    1024 + 4 slot (K) and 1088 + 4 slot (V)."""
    shape = O.Shape(num_kv_heads=1, num_q_heads=1, sink=16, recent=16, group=128)
    cache = O.new_cache(shape, num_pages=4, num_slots=1)
    assert cache.pages.shape == (4, 1, 1152)
    eye = np.zeros((1, 128, 128), np.uint16)
    eye[0, np.arange(128), np.arange(128)] = 0x3F80
    layer = O.Layer(eye, eye, np.float32(case["clip"]), np.float32(case["clip"]))
    sign = np.array([(-1) ** bin(case["k"] & i).count("1") for i in range(128)], np.float64)
    x = O.f64_to_bf16(sign)[None, None]
    k, v = (x, None) if case["kind"] == "K" else (None, x)
    O.kv_write(shape, cache, layer, k, v, [0], [16 + case["slot"]], np.array([[0, 1, 2, 3]], np.int32), [64])
    blk = cache.pages[1, 0]
    p = case["params"]
    spike_group = [p[0:2], p[2:4]][0 if p[0] else 1]            # (s, z) of the group holding the spike
    if case["kind"] == "K":
        codes = blk[0:512].copy()
        assert codes[case["index"]] == case["value"]
        codes[case["index"]] = 0
        assert codes.sum() == 0
        off = 1024 + 4 * case["slot"]
    else:
        words = blk[512:1024].copy().view("<u4")
        assert words[case["index"]] == case["value"]
        words[case["index"]] = 0
        assert words.sum() == 0
        off = 1088 + 4 * case["slot"]
    assert list(blk[off:off + 4].view("<u2")) == spike_group
    rest = np.ones(1152, bool)
    rest[0:1024] = False
    rest[off:off + 4] = False
    assert blk[rest].sum() == 0


def test_reconstruction_within_half_a_step():
    """kv_write then the read path's dequantisation: every rotated value of an
    unclipped token is recovered within s/2 plus fp16 rounding of z, with s the
    token's single scale."""
    rng = np.random.default_rng(3)
    shape = O.Shape(num_kv_heads=2, num_q_heads=2, group=128)
    layer = random_layer(rng, 2)
    layer = O.Layer(layer.u_k, layer.u_v, np.float32(1e4), np.float32(1e4))   # no clipping
    L = 300
    table = np.arange(20, dtype=np.int32)[None]
    cache = O.new_cache(shape, 20, 1)
    k = synth.f32_to_bf16_bits(rng.standard_normal((L, 2, 128)))
    info = O.kv_write(shape, cache, layer, k, None, np.zeros(L, int), np.arange(L), table, [L])
    d = info["K"]
    for i, p in enumerate(d["token"]):        # the INT2 tokens (pos >= sink), pos = p here
        pid, t = table[0, p // 16], p % 16
        for h in range(2):
            blk = cache.pages[pid, h]
            codes = O.unpack_k_codes(blk[32 * t:32 * t + 32]).astype(np.float64)
            s16, z16 = blk[1024 + 4 * t:1028 + 4 * t].view("<f2").astype(np.float64)
            got = z16 + s16 * codes
            dz = abs(z16 - d["z_pre"][i, h, 0])
            assert s16 == d["s16"][i, h, 0] and (np.abs(got - d["w"][i, h]) <= s16 / 2 + dz + 1e-12).all()


def test_decode_brute_force_over_reconstructed_keys():
    """decode over a 128-group cache equals softmax attention, with explicit loops,
    over the keys and values the page bytes decode to (sink and ring rows exact)."""
    rng = np.random.default_rng(4)
    shape = O.Shape(num_kv_heads=1, num_q_heads=2, group=128)
    layer = random_layer(rng, 1)
    L = 900
    table = rng.permutation(60).astype(np.int32)[None]
    cache = O.new_cache(shape, 60, 1)
    k = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128)))
    v = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128)))
    O.kv_write(shape, cache, layer, k, v, np.zeros(L, int), np.arange(L), table, [L])
    q = synth.f32_to_bf16_bits(rng.standard_normal((1, 2, 128)))
    out = O.decode(shape, cache, layer, q, table, [L], SIG)
    # keys and values as stored: BF16 rows for sink and recent, INT2 rows decoded by hand
    R_k, R_v = O.rotation(layer.u_k[0]), O.rotation(layer.u_v[0])
    K, V = O.bf16_to_f64(k[:, 0]).copy(), O.bf16_to_f64(v[:, 0]).copy()
    for p in range(64, L - 256):
        blk = cache.pages[table[0, p // 16], 0]
        t = p % 16
        kc = O.unpack_k_codes(blk[32 * t:32 * t + 32]).astype(np.float64)
        ks, kz = blk[1024 + 4 * t:1028 + 4 * t].view("<f2").astype(np.float64)
        vc = ((blk[512:1024].view("<u4") >> (2 * t)) & 3).astype(np.float64)
        vs, vz = blk[1088 + 4 * t:1092 + 4 * t].view("<f2").astype(np.float64)
        K[p] = (kz + ks * kc) @ R_k.T
        V[p] = (vz + vs * vc) @ R_v.T
    for hq in range(2):
        ref = brute_attention(O.bf16_to_f64(q[0, hq]), K, V, SIG)
        assert np.abs(out[0, hq] - ref).max() < 1e-10
