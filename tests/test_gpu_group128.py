"""GPU parity of the 128-channel-group format (one fp16 scale and zero per token
and head, 1152-byte page blocks: 2.25 bits per element, the format behind the
Russian page's paragraph 4 "2.28 bits per KV element") against the oracle,
under the same parity rules as the 64-channel format (gpu_harness): kv_write
bytes bit-exact up to excused near-ties, decode / extend / cascade outputs
within the decode tolerance."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import synth
from test_gpu_cascade import run_cascade, shared_cache
from test_gpu_extend import fill_prefix, run_extend
from test_gpu_parity import make_layer, run_scenario

pytestmark = pytest.mark.gpu


def test_tiny_1k_write_and_decode(gpu):
    rng = np.random.default_rng(0)
    shape = O.Shape(num_kv_heads=1, num_q_heads=4, group=128)
    law = synth.outlier_law(rng, 1)
    layer = make_layer(rng, shape, law, 2048)
    L = 1024
    stats, res = run_scenario(gpu, shape, layer, law, [L], synth.contiguous_page_table(1, 64),
                              [(np.zeros(L), np.arange(L))], rng)
    print("write stats", stats, "decode", res, flush=True)
    assert stats[0]["codes"] == 2 * 960 * 128


@pytest.mark.parametrize("G", [1, 3, 4, 8])
def test_ragged_batch_permuted_pages(gpu, G):
    rng = np.random.default_rng(20 + G)
    shape = O.Shape(num_kv_heads=2, num_q_heads=2 * G, group=128)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [0, 1, 63, 64, 65, 320, 321, 333, 1000, 2049]
    table = synth.permuted_page_table(rng, len(lens), 130)
    seq_idx = np.concatenate([np.full(L, s) for s, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L) for L in lens])
    perm = rng.permutation(len(pos))
    stats, res = run_scenario(gpu, shape, layer, law, lens, table, [(seq_idx[perm], pos[perm])], rng)
    print("G", G, "decode", res, flush=True)


def test_chunked_and_single_token_writes(gpu):
    rng = np.random.default_rng(21)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8, group=128)
    law = synth.heavy_tail_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    table = synth.permuted_page_table(rng, 1, 40)
    calls = [(np.zeros(100), np.arange(100)), (np.zeros(257), np.arange(100, 357))]
    calls += [([0], [p]) for p in range(357, 400)]
    stats, res = run_scenario(gpu, shape, layer, law, [400], table, calls, rng)
    print("decode", res, flush=True)


@pytest.mark.parametrize("G", [4, 8])
def test_many_pairs_plan(gpu, G):
    """8 sequences x 4 KV heads: the many-pairs plan (stored query records)."""
    rng = np.random.default_rng(22 + G)
    shape = O.Shape(num_kv_heads=4, num_q_heads=4 * G, group=128)
    law = synth.outlier_law(rng, 4)
    layer = make_layer(rng, shape, law, 256)
    lens = [700, 1500, 321, 2000, 64, 999, 1234, 3000]
    table = synth.permuted_page_table(rng, len(lens), 190)
    seq_idx = np.concatenate([np.full(L, s) for s, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L) for L in lens])
    stats, res = run_scenario(gpu, shape, layer, law, lens, table, [(seq_idx, pos)], rng, check_each_call=False)
    print("G", G, "decode", res, flush=True)


@pytest.mark.parametrize("sink,recent", [(0, 1), (16, 5), (64, 256)])
def test_nan_poisoned_unwritten_slots(gpu, sink, recent):
    rng = np.random.default_rng(600 + sink + recent)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8, sink=sink, recent=recent, group=128)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [1, 17, sink + recent + 3, 333, 700]
    table = synth.permuted_page_table(rng, len(lens), 50)
    calls = [(np.full(L, s), np.arange(L)) for s, L in enumerate(lens)]
    stats, res = run_scenario(gpu, shape, layer, law, lens, table, calls, rng, poison=True)
    print(sink, recent, "poisoned decode", res, flush=True)


@pytest.mark.parametrize("G", [2, 8])
def test_extend(gpu, G):
    rng = np.random.default_rng(60 + G)
    shape = O.Shape(num_kv_heads=2, num_q_heads=2 * G, group=128)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    prefix = [0, 63, 321, 1000, 2049, 6500]
    chunks = [5, 17, 3, 40, 33, 9]
    table = synth.permuted_page_table(rng, len(prefix), 420)
    cache = O.new_cache(shape, int(table.max()) + 1, len(prefix))
    fill_prefix(shape, cache, layer, law, rng, prefix, table)
    res, *_ = run_extend(gpu, shape, cache, layer, law, rng, prefix, chunks, table)
    print("G", G, "extend", res, flush=True)


@pytest.mark.parametrize("G", [4, 8])
def test_cascade(gpu, G):
    rng = np.random.default_rng(75 + G)
    shape = O.Shape(num_kv_heads=2, num_q_heads=2 * G, group=128)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [3001, 2500, 1800, 1200, 900, 2049]
    groups = [(0, 3, 64 + 16 * 100), (3, 5, 64 + 16 * 37)]
    cache, table = shared_cache(shape, layer, law, rng, lens, groups, 200)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0, 3, 5], [100, 37], 3, 100, rng)
    print("G", G, "cascade", res, "vs decode_attn", d, flush=True)
