"""Pins of the oracle's all-BF16 paged decode (the baseline the pages compare
OSCAR against: Italian page "Velocita di decodifica", Spanish summary section
4).  Layout positions written as literal numbers, round trip through a
permuted table, brute force with explicit loops, closed forms (L = 1, equal
keys), agreement with the mixed-cache oracle where that one reads only BF16
tokens (L <= sink + recent), and page-table invariance."""
import math

import numpy as np
import pytest

import oracle as O
import synth
from test_oracle_attention import brute_attention

SIG = 1 / math.sqrt(128)


def tokens(rng, L, H):
    k = synth.f32_to_bf16_bits(rng.standard_normal((L, H, 128)))
    v = synth.f32_to_bf16_bits(rng.standard_normal((L, H, 128)))
    return k, v


def test_layout_positions_literal():
    """Token at position 17 of sequence 0 lives in slot 1 of logical page 1:
    K channel 5 at element 133 (= 128 + 5), V channel 5 at element 2129
    (= 2048 + 80 + 1), V channel 127 at 4081."""
    rng = np.random.default_rng(3)
    table = np.array([[4, 2, 7]], np.int32)
    pages = O.new_bf16_pages(8, 2)
    k, v = tokens(rng, 20, 2)
    O.bf16_pages_write(pages, k, v, np.zeros(20, int), np.arange(20), table)
    for h in range(2):
        assert pages[2, h, 133] == k[17, h, 5]
        assert pages[2, h, 2129] == v[17, h, 5]
        assert pages[2, h, 4081] == v[17, h, 127]
        assert pages[4, h, 0] == k[0, h, 0]
        assert pages[4, h, 2048 + 15] == v[15, h, 0]
    assert (pages[[0, 1, 3, 5, 6, 7]] == 0).all()   # untouched pages
    assert (pages[2, :, 128 * 4:2048] == 0).all()   # slots 4..15 of page 2: past position 19


def test_gather_round_trip_permuted():
    rng = np.random.default_rng(4)
    L, H = 100, 3
    table = rng.permutation(16).astype(np.int32)[None, :7]
    pages = O.new_bf16_pages(16, H)
    k, v = tokens(rng, L, H)
    O.bf16_pages_write(pages, k, v, np.zeros(L, int), np.arange(L), table)
    for h in range(H):
        K, V = O.bf16_pages_gather(pages, table, 0, h, L)
        assert np.array_equal(K, O.bf16_to_f64(k[:, h]))
        assert np.array_equal(V, O.bf16_to_f64(v[:, h]))


@pytest.mark.parametrize("L", [1, 5, 16, 17, 40])
def test_brute_force(L):
    rng = np.random.default_rng(L + 100)
    H, G = 2, 2
    table = np.arange(3, dtype=np.int32)[None]
    pages = O.new_bf16_pages(3, H)
    k, v = tokens(rng, L, H)
    O.bf16_pages_write(pages, k, v, np.zeros(L, int), np.arange(L), table)
    q = synth.decode_queries(rng, 1, H * G)
    out = O.decode_bf16_paged(pages, q, table, [L], H, SIG)
    for hq in range(H * G):
        h = hq // G
        ref = brute_attention(O.bf16_to_f64(q[0, hq]), O.bf16_to_f64(k[:, h]), O.bf16_to_f64(v[:, h]), SIG)
        assert np.abs(out[0, hq] - ref).max() < 1e-12


def test_length_one_and_zero():
    rng = np.random.default_rng(5)
    table = np.arange(2, dtype=np.int32)[None]
    pages = O.new_bf16_pages(2, 1)
    k, v = tokens(rng, 1, 1)
    O.bf16_pages_write(pages, k, v, [0], [0], table)
    q = synth.decode_queries(rng, 1, 4)
    out = O.decode_bf16_paged(pages, q, table, [1], 1, SIG)
    for hq in range(4):
        assert np.array_equal(out[0, hq], O.bf16_to_f64(v[0, 0]))
    assert (O.decode_bf16_paged(pages, q, table, [0], 1, SIG) == 0).all()


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(6)
    L = 300
    table = np.arange(19, dtype=np.int32)[None]
    pages = O.new_bf16_pages(19, 1)
    _, v = tokens(rng, L, 1)
    k = np.tile(synth.f32_to_bf16_bits(rng.standard_normal((1, 1, 128))), (L, 1, 1))
    O.bf16_pages_write(pages, k, v, np.zeros(L, int), np.arange(L), table)
    q = synth.decode_queries(rng, 1, 1)
    out = O.decode_bf16_paged(pages, q, table, [L], 1, SIG)
    assert np.abs(out[0, 0] - O.bf16_to_f64(v[:, 0]).mean(axis=0)).max() < 1e-12


@pytest.mark.parametrize("L", [64, 250, 320])
def test_matches_mixed_cache_oracle_on_bf16_lengths(L):
    """For L <= sink + recent the mixed cache holds every token in BF16 (sink
    rows and ring), so its oracle and the paged BF16 oracle read the same
    values through different layouts."""
    rng = np.random.default_rng(L)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    table = np.arange(20, dtype=np.int32)[None]
    k, v = tokens(rng, L, 2)
    cache = O.new_cache(shape, 20, 1)
    layer = O.Layer(np.zeros((2, 128, 128), np.uint16), np.zeros((2, 128, 128), np.uint16),
                    np.float32(1.0), np.float32(1.0))
    O.kv_write(shape, cache, layer, k, v, np.zeros(L, int), np.arange(L), table, [L])
    pages = O.new_bf16_pages(20, 2)
    O.bf16_pages_write(pages, k, v, np.zeros(L, int), np.arange(L), table)
    q = synth.decode_queries(rng, 1, 8)
    a = O.decode(shape, cache, layer, q, table, [L], SIG)
    b = O.decode_bf16_paged(pages, q, table, [L], 2, SIG)
    assert np.abs(a - b).max() < 1e-12


def test_page_table_invariance_two_sequences():
    rng = np.random.default_rng(8)
    H, lens = 2, [70, 33]
    k0, v0 = tokens(rng, 70, H)
    k1, v1 = tokens(rng, 33, H)
    q = synth.decode_queries(rng, 2, 2 * H)
    outs = []
    for table in (np.array([[0, 1, 2, 3, 4], [5, 6, 7, 8, 9]], np.int32),
                  rng.permutation(12).astype(np.int32)[:10].reshape(2, 5)):
        pages = O.new_bf16_pages(12, H)
        O.bf16_pages_write(pages, k0, v0, np.zeros(70, int), np.arange(70), table)
        O.bf16_pages_write(pages, k1, v1, np.ones(33, int), np.arange(33), table)
        outs.append(O.decode_bf16_paged(pages, q, table, lens, H, SIG))
    assert np.array_equal(outs[0], outs[1])
