"""Pins of the oracle's extend (chunked-prefill) attention, each against
something other than the function itself: brute-force causal attention with
explicit loops where the prefix holds no INT2 token, pure causal
self-attention for an empty prefix, causality (later chunk tokens cannot move
earlier outputs), and a chunk key whose logit underflows, which reduces the
query's attention to the oracle's decode over the stored prefix (pinned in
test_oracle_attention.py).  Read path: the Italian page's section
"Architettura del Sistema di Serving e Layout di Memoria"; the Spanish
summary, 2.2 B."""
import math

import numpy as np
import pytest

import oracle as O
import synth
from test_oracle_attention import brute_attention, random_layer

SIG = 1 / math.sqrt(128)


def bf16(rng, *shape):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape))


def prefix_cache(shape, rng, L, table, layer):
    cache = O.new_cache(shape, num_pages=int(table.max()) + 1, num_slots=1)
    k = bf16(rng, max(L, 1), shape.num_kv_heads, 128)[:L]
    v = bf16(rng, max(L, 1), shape.num_kv_heads, 128)[:L]
    if L:
        O.kv_write(shape, cache, layer, k, v, np.zeros(L, int), np.arange(L), table, [L])
    return cache, k, v


@pytest.mark.parametrize("L,T", [(0, 5), (10, 7), (64, 3), (150, 20), (300, 4)])
def test_bf16_only_prefix_equals_brute_force_causal(L, T):
    """L_prev + T small enough that the prefix holds no INT2 token (L_prev <=
    sink + recent): every key is a bf16 input, so each chunk query's output is
    plain causal softmax attention over prefix + chunk tokens 0..i."""
    rng = np.random.default_rng(100 + L + T)
    shape = O.Shape(num_kv_heads=1, num_q_heads=2)
    table = np.arange(30, dtype=np.int32)[None]
    layer = random_layer(rng, 1)
    cache, k, v = prefix_cache(shape, rng, L, table, layer)
    q = bf16(rng, T, 2, 128)
    kn, vn = bf16(rng, T, 1, 128), bf16(rng, T, 1, 128)
    out = O.extend(shape, cache, layer, q, kn, vn, [0, T], [L], table, SIG)
    K = np.concatenate([O.bf16_to_f64(k[:, 0]), O.bf16_to_f64(kn[:, 0])])
    V = np.concatenate([O.bf16_to_f64(v[:, 0]), O.bf16_to_f64(vn[:, 0])])
    for i in range(T):
        for hq in range(2):
            ref = brute_attention(O.bf16_to_f64(q[i, hq]), K[:L + i + 1], V[:L + i + 1], SIG)
            assert np.abs(out[i, hq] - ref).max() < 1e-12


def test_first_query_of_empty_prefix_returns_its_value():
    rng = np.random.default_rng(3)
    shape = O.Shape(num_kv_heads=2, num_q_heads=4)
    table = np.zeros((2, 4), np.int32)
    layer = random_layer(rng, 2)
    cache = O.new_cache(shape, 1, 2)
    q = bf16(rng, 6, 4, 128)
    kn, vn = bf16(rng, 6, 2, 128), bf16(rng, 6, 2, 128)
    out = O.extend(shape, cache, layer, q, kn, vn, [0, 2, 6], [0, 0], table, SIG)
    for t0 in (0, 2):            # the first token of each chunk sees only itself
        for hq in range(4):
            assert np.array_equal(out[t0, hq], O.bf16_to_f64(vn[t0, hq // 2]))


def test_causality_later_tokens_do_not_move_earlier_outputs():
    rng = np.random.default_rng(4)
    shape = O.Shape(num_kv_heads=1, num_q_heads=4)
    L, T = 700, 9
    table = rng.permutation(50).astype(np.int32)[None]
    layer = random_layer(rng, 1)
    cache, _, _ = prefix_cache(shape, rng, L, table, layer)
    q = bf16(rng, T, 4, 128)
    kn, vn = bf16(rng, T, 1, 128), bf16(rng, T, 1, 128)
    a = O.extend(shape, cache, layer, q, kn, vn, [0, T], [L], table, SIG)
    kn2, vn2 = kn.copy(), vn.copy()
    kn2[5:], vn2[5:] = bf16(rng, T - 5, 1, 128), bf16(rng, T - 5, 1, 128)
    b = O.extend(shape, cache, layer, q, kn2, vn2, [0, T], [L], table, SIG)
    assert np.array_equal(a[:5], b[:5])
    assert not np.array_equal(a[5:], b[5:])


@pytest.mark.parametrize("L", [321, 1000, 2049])
def test_underflowing_chunk_key_leaves_the_decode_of_the_stored_prefix(L):
    """A single chunk token whose key is -64 q (bf16-exact) has logit
    -64 |q|^2 / sqrt(128), far below every prefix logit: exp underflows to 0
    in fp64, so the query attends to the stored prefix alone -- the oracle's
    decode of a sequence of length L_prev, INT2 history included."""
    rng = np.random.default_rng(L)
    shape = O.Shape(num_kv_heads=1, num_q_heads=1)
    table = rng.permutation(140).astype(np.int32)[None]
    layer = random_layer(rng, 1)
    cache, _, _ = prefix_cache(shape, rng, L, table, layer)
    q = bf16(rng, 1, 1, 128)
    kn = O.f64_to_bf16(-64.0 * O.bf16_to_f64(q[:, :1]))     # exact: a power-of-two multiple
    assert np.array_equal(O.bf16_to_f64(kn), -64.0 * O.bf16_to_f64(q[:, :1]))
    vn = bf16(rng, 1, 1, 128)
    out = O.extend(shape, cache, layer, q, kn, vn, [0, 1], [L], table, SIG)
    ref = O.decode(shape, cache, layer, q, table, [L], SIG)
    assert np.abs(out[0, 0] - ref[0, 0]).max() < 1e-12


def test_two_sequences_are_independent():
    """Chunks of two sequences in one call equal two single-sequence calls."""
    rng = np.random.default_rng(5)
    shape = O.Shape(num_kv_heads=1, num_q_heads=2)
    table = np.stack([rng.permutation(60), 60 + rng.permutation(60)]).astype(np.int32)
    layer = random_layer(rng, 1)
    cache = O.new_cache(shape, 120, 2)
    for b, L in enumerate((500, 333)):
        k, v = bf16(rng, L, 1, 128), bf16(rng, L, 1, 128)
        O.kv_write(shape, cache, layer, k, v, np.full(L, b), np.arange(L), table, [500, 333])
    q = bf16(rng, 7, 2, 128)
    kn, vn = bf16(rng, 7, 1, 128), bf16(rng, 7, 1, 128)
    both = O.extend(shape, cache, layer, q, kn, vn, [0, 3, 7], [500, 333], table, SIG)
    one = O.extend(shape, cache, layer, q[:3], kn[:3], vn[:3], [0, 3, 3], [500, 333], table, SIG)
    two = O.extend(shape, cache, layer, q[3:], kn[3:], vn[3:], [0, 0, 4], [500, 333], table, SIG)
    assert np.array_equal(both[:3], one)
    assert np.array_equal(both[3:], two)
