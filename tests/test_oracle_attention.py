"""Pins of the oracle's decode attention: brute force on tiny inputs, closed
forms (L = 1, equal keys), a hand-built INT2 page whose inverse rotation has a
closed form (rows of the Hadamard matrix from scipy), the folded form, and
page-table invariance.  Region rule: Italian page "Architettura del Sistema di
Serving e Layout di Memoria"; read path: same section and Spanish summary 2.2 B."""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle as O
import synth

SIG = 1 / math.sqrt(128)


def brute_attention(q, K, V, scale):
    """Explicit loops with math.exp."""
    lg = [scale * sum(q[c] * K[i][c] for c in range(len(q))) for i in range(len(K))]
    m = max(lg)
    w = [math.exp(x - m) for x in lg]
    tot = sum(w)
    return np.array([sum(w[i] * V[i][c] for i in range(len(K))) / tot for c in range(len(q))])


def random_layer(rng, H):
    U = np.stack([O.f64_to_bf16(np.linalg.qr(rng.standard_normal((128, 128)))[0]) for _ in range(H)])
    U2 = np.stack([O.f64_to_bf16(np.linalg.qr(rng.standard_normal((128, 128)))[0]) for _ in range(H)])
    return O.Layer(U, U2, np.float32(3.5), np.float32(3.5))


def fill(shape, rng, L, table, n_slots=1, seq=0):
    cache = O.new_cache(shape, num_pages=int(table.max()) + 1, num_slots=n_slots)
    layer = random_layer(rng, shape.num_kv_heads)
    k = synth.f32_to_bf16_bits(rng.standard_normal((L, shape.num_kv_heads, 128)))
    v = synth.f32_to_bf16_bits(rng.standard_normal((L, shape.num_kv_heads, 128)))
    O.kv_write(shape, cache, layer, k, v, np.full(L, seq), np.arange(L), table, [L] * n_slots)
    return cache, layer, k, v


@pytest.mark.parametrize("L", [1, 17, 64, 65, 200, 320])
def test_bf16_only_lengths_equal_brute_force(L):
    """L <= 320 touches no INT2 token: exact softmax attention on the bf16 inputs."""
    rng = np.random.default_rng(L)
    shape = O.Shape(num_kv_heads=1, num_q_heads=2)
    table = np.arange(20, dtype=np.int32)[None]
    cache, layer, k, v = fill(shape, rng, L, table)
    q = synth.decode_queries(rng, 1, 2)
    out = O.decode(shape, cache, layer, q, table, [L], SIG)
    K = O.bf16_to_f64(k[:, 0])
    V = O.bf16_to_f64(v[:, 0])
    for hq in range(2):
        ref = brute_attention(O.bf16_to_f64(q[0, hq]), K, V, SIG)
        assert np.abs(out[0, hq] - ref).max() < 1e-12


def test_length_one_returns_v0_and_zero_length_zeros():
    rng = np.random.default_rng(9)
    shape = O.Shape(num_kv_heads=1, num_q_heads=1)
    table = np.arange(4, dtype=np.int32)[None]
    cache, layer, k, v = fill(shape, rng, 1, table)
    q = synth.decode_queries(rng, 1, 1)
    assert np.array_equal(O.decode(shape, cache, layer, q, table, [1], SIG)[0, 0], O.bf16_to_f64(v[0, 0]))
    assert (O.decode(shape, cache, layer, q, table, [0], SIG) == 0).all()


def test_equal_keys_give_mean_of_values():
    """All keys identical (zero vector, so the INT2 history decodes it
    exactly) -> uniform attention -> the mean of the reconstructed values."""
    rng = np.random.default_rng(10)
    shape = O.Shape(num_kv_heads=1, num_q_heads=1)
    L = 700
    table = np.arange(50, dtype=np.int32)[None]
    cache = O.new_cache(shape, 50, 1)
    layer = random_layer(rng, 1)
    k = np.zeros((L, 1, 128), np.uint16)
    v = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128)))
    O.kv_write(shape, cache, layer, k, v, np.zeros(L, int), np.arange(L), table, [L])
    q = synth.decode_queries(rng, 1, 1)
    out = O.decode(shape, cache, layer, q, table, [L], SIG)
    _, V, _ = O.gather_sequence(shape, cache, layer, 0, 0, L, table)
    assert np.abs(out[0, 0] - V.mean(0)).max() < 1e-12


def test_hand_built_int2_page_closed_form():
    """INT2 slots written by hand: K slot t has code 1 at channel j_t (s=1, z=0),
    V slot t has code 2 at channel m_t (s=0.5, z=0.25).  With U = I,
    k_hat = e_j P H = row br(j) of H and v_hat = 0.25*sqrt(128) e_0 + row br(m)
    of H.  H rows come from scipy's Sylvester construction."""
    rng = np.random.default_rng(11)
    shape = O.Shape(num_kv_heads=1, num_q_heads=2, sink=16, recent=16)
    L = 48                                   # sink [0,16) INT2 [16,32) recent [32,48)
    table = np.array([[3, 0, 2]], np.int32)  # logical page 1 -> physical 0
    cache = O.new_cache(shape, 4, 1)
    eye = np.zeros((1, 128, 128), np.uint16)
    eye[0, np.arange(128), np.arange(128)] = 0x3F80
    layer = O.Layer(eye, eye, np.float32(10), np.float32(10))
    ks = synth.f32_to_bf16_bits(rng.standard_normal((16, 128)))
    vs = synth.f32_to_bf16_bits(rng.standard_normal((16, 128)))
    kr = synth.f32_to_bf16_bits(rng.standard_normal((16, 128)))
    vr = synth.f32_to_bf16_bits(rng.standard_normal((16, 128)))
    cache.k_sink[0, 0] = ks
    cache.v_sink[0, 0] = vs
    cache.k_ring[0, 0, np.arange(32, 48) % 16] = kr
    cache.v_ring[0, 0, np.arange(32, 48) % 16] = vr
    j = rng.integers(0, 128, 16)
    m = rng.integers(0, 128, 16)
    blk = cache.pages[0, 0]
    words = np.zeros(128, np.uint32)
    for t in range(16):
        blk[32 * t + j[t] // 4] = 1 << (2 * (j[t] % 4))
        words[m[t]] |= np.uint32(2 << (2 * t))
        blk[1024 + 8 * t:1024 + 8 * t + 8] = np.array([0x3C00, 0, 0x3C00, 0], "<u2").view(np.uint8)
        blk[1152 + 8 * t:1152 + 8 * t + 8] = np.array([0x3800, 0x3400, 0x3800, 0x3400], "<u2").view(np.uint8)
    blk[512:1024] = words.astype("<u4").view(np.uint8)
    Hs = scipy.linalg.hadamard(128) / math.sqrt(128)
    br = [int(format(i, "07b")[::-1], 2) for i in range(128)]
    Kx = [O.bf16_to_f64(r) for r in ks] + [Hs[br[j[t]]] for t in range(16)] + [O.bf16_to_f64(r) for r in kr]
    Vx = [O.bf16_to_f64(r) for r in vs] + \
         [0.25 * math.sqrt(128) * np.eye(128)[0] + Hs[br[m[t]]] for t in range(16)] + \
         [O.bf16_to_f64(r) for r in vr]
    q = synth.decode_queries(rng, 1, 2)
    out = O.decode(shape, cache, layer, q, table, [L], SIG)
    for hq in range(2):
        ref = brute_attention(O.bf16_to_f64(q[0, hq]), Kx, Vx, SIG)
        assert np.abs(out[0, hq] - ref).max() < 1e-12


def test_folded_equals_unfolded():
    rng = np.random.default_rng(12)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    L = 1000
    table = np.stack([rng.permutation(64)]).astype(np.int32)
    cache, layer, k, v = fill(shape, rng, L, table)
    q = synth.decode_queries(rng, 1, 8)
    a = O.decode(shape, cache, layer, q, table, [L], SIG)
    b = O.decode_folded(shape, cache, layer, q, table, [L], SIG)
    assert np.abs(a - b).max() < 1e-10


def test_page_permutation_invariance():
    rng = np.random.default_rng(13)
    shape = O.Shape(num_kv_heads=1, num_q_heads=4)
    L = 777
    t1 = np.arange(49, dtype=np.int32)[None]
    t2 = rng.permutation(60)[:49].astype(np.int32)[None]
    layer = random_layer(rng, 1)
    k = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128)))
    v = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128)))
    outs = []
    for t in (t1, t2):
        cache = O.new_cache(shape, 60, 1)
        O.kv_write(shape, cache, layer, k, v, np.zeros(L, int), np.arange(L), t, [L])
        outs.append(O.decode(shape, cache, layer, synth.decode_queries(np.random.default_rng(0), 1, 4), t, [L], SIG))
    assert np.array_equal(outs[0], outs[1])


def test_chunked_writes_equal_one_write():
    """Writing a sequence token by token (decode steps, growing L_after) leaves
    the same cache as one prefill write of all tokens."""
    rng = np.random.default_rng(14)
    shape = O.Shape(num_kv_heads=1, num_q_heads=1, sink=16, recent=32)
    L = 150
    table = np.arange(10, dtype=np.int32)[None]
    layer = random_layer(rng, 1)
    k = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128)))
    v = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128)))
    c1 = O.new_cache(shape, 10, 1)
    O.kv_write(shape, c1, layer, k, v, np.zeros(L, int), np.arange(L), table, [L])
    c2 = O.new_cache(shape, 10, 1)
    O.kv_write(shape, c2, layer, k[:100], v[:100], np.zeros(100, int), np.arange(100), table, [100])
    for p in range(100, L):
        O.kv_write(shape, c2, layer, k[p:p + 1], v[p:p + 1], [0], [p], table, [p + 1])
    assert np.array_equal(c1.pages, c2.pages)
    assert np.array_equal(c1.k_sink, c2.k_sink)
    # ring rows of the last 32 positions agree (older rows may differ: they are dead)
    rows = np.arange(L - 32, L) % 32
    assert np.array_equal(c1.k_ring[0, 0, rows], c2.k_ring[0, 0, rows])
    q = synth.decode_queries(rng, 1, 1)
    assert np.array_equal(O.decode(shape, c1, layer, q, table, [L], SIG),
                          O.decode(shape, c2, layer, q, table, [L], SIG))
