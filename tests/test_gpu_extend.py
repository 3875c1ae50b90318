"""GPU parity of extend (chunked-prefill) attention against the oracle's
extend: chunk queries over the stored prefix (sink and ring rows in BF16, INT2
history through the folded rotation) and causally over the chunk's own BF16
keys.  Read path: the Italian page's section "Architettura del Sistema di
Serving e Layout di Memoria"; the Spanish summary, 2.2 B.  Outputs are held to
the decode tolerance (bf16 units, written out in gpu_harness)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import synth
from gpu_harness import (SIG, compare_outputs, device_cache, from_dev_bf16, host_cache, lib_shape, to_dev_bf16,
                         to_dev_i32)
from test_gpu_parity import make_layer

pytestmark = pytest.mark.gpu


def fill_prefix(shape, cache, layer, law, rng, prefix_lens, table):
    """Oracle-written prefixes: sequence s holds prefix_lens[s] tokens of `law`."""
    seq = np.concatenate([np.full(L, s) for s, L in enumerate(prefix_lens)] + [np.zeros(0, int)])
    pos = np.concatenate([np.arange(L) for L in prefix_lens] + [np.zeros(0, int)])
    if len(seq):
        k = np.concatenate([law.sample_bf16(rng, L) for L in prefix_lens])
        v = np.concatenate([law.sample_bf16(rng, L) for L in prefix_lens])
        O.kv_write(shape, cache, layer, k, v, seq, pos, table, list(prefix_lens))


def run_extend(device, shape, cache, layer, law, rng, prefix_lens, chunk_lens, table, max_chunk=None,
               dc=None):
    """One extend call over `cache` (oracle-written unless `dc`, the device copy, is
    given); returns (errors, q, k, v) with the chunk's bf16 inputs."""
    import torch
    import int2_rotated_kv_write_amd as lib
    T = int(sum(chunk_lens))
    cu = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    max_chunk = max_chunk or max(max(chunk_lens), 1)
    q = synth.decode_queries(rng, T, shape.num_q_heads)
    k = law.sample_bf16(rng, T)
    v = law.sample_bf16(rng, T)
    want = O.extend(shape, cache, layer, q, k, v, cu, prefix_lens, table, SIG)
    ls = lib_shape(shape)
    if dc is None:
        dc = device_cache(shape, cache, layer, device)
    ws = torch.empty(lib.extend_workspace_bytes(ls, T, table.shape[1], max_chunk), dtype=torch.uint8,
                     device=device)
    ws.fill_(0xFF)   # nothing the call reads may come from a previous workspace content
    out = torch.full((T, shape.num_q_heads, 128), float("nan"), dtype=torch.bfloat16, device=device)
    lib.extend_attn(ls, dc, to_dev_bf16(q, device), to_dev_bf16(k, device), to_dev_bf16(v, device),
                    to_dev_i32(cu, device), to_dev_i32(prefix_lens, device), to_dev_i32(table, device), out, ws,
                    max_chunk, SIG)
    torch.cuda.synchronize()
    return compare_outputs(from_dev_bf16(out), want), q, k, v


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_ragged_prefixes_and_chunks(gpu, G):
    """Eight sequences in one call: prefixes at the region edges (empty, inside
    the sink, at sink + recent, one INT2 token, several ranges of INT2 pages)
    with chunks of 1 to 64 tokens; random disjoint page tables."""
    rng = np.random.default_rng(40 + G)
    shape = O.Shape(num_kv_heads=2, num_q_heads=2 * G)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    prefix = [0, 1, 63, 320, 321, 1000, 2049, 6500]
    chunks = [5, 1, 17, 64, 3, 40, 33, 9]
    max_pages = 420                     # 416 INT2 pages: two ranges
    table = synth.permuted_page_table(rng, len(prefix), max_pages)
    cache = O.new_cache(shape, int(table.max()) + 1, len(prefix))
    fill_prefix(shape, cache, layer, law, rng, prefix, table)
    res, *_ = run_extend(gpu, shape, cache, layer, law, rng, prefix, chunks, table)
    print("G", G, "extend", res, flush=True)


def test_long_chunk(gpu):
    """One 300-token chunk over a 3,000-token prefix, G = 4: 75 tiles of 16
    query heads share each INT2 page read; the causal BF16 part spans up to
    620 keys."""
    rng = np.random.default_rng(7)
    shape = O.Shape(num_kv_heads=1, num_q_heads=4)
    law = synth.outlier_law(rng, 1)
    layer = make_layer(rng, shape, law, 256)
    table = synth.permuted_page_table(rng, 1, 200)
    cache = O.new_cache(shape, int(table.max()) + 1, 1)
    fill_prefix(shape, cache, layer, law, rng, [3000], table)
    res, *_ = run_extend(gpu, shape, cache, layer, law, rng, [3000], [300], table)
    print("long chunk", res, flush=True)


def test_empty_chunks_and_max_chunk_slack(gpu):
    """Sequences with no chunk tokens between others, and max_chunk above the
    longest chunk (grids larger than the work)."""
    rng = np.random.default_rng(8)
    shape = O.Shape(num_kv_heads=2, num_q_heads=4)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    prefix = [500, 0, 900, 40]
    chunks = [0, 7, 0, 12]
    table = synth.permuted_page_table(rng, 4, 64)
    cache = O.new_cache(shape, int(table.max()) + 1, 4)
    fill_prefix(shape, cache, layer, law, rng, prefix, table)
    res, *_ = run_extend(gpu, shape, cache, layer, law, rng, prefix, chunks, table, max_chunk=50)
    print("empty chunks", res, flush=True)


def test_zero_tokens_is_a_no_op(gpu):
    import torch
    import int2_rotated_kv_write_amd as lib
    shape = O.Shape(num_kv_heads=1, num_q_heads=2)
    ls = lib_shape(shape)
    layer = O.Layer(np.zeros((1, 128, 128), np.uint16), np.zeros((1, 128, 128), np.uint16),
                    np.float32(1), np.float32(1))
    dc = device_cache(shape, O.new_cache(shape, 4, 1), layer, gpu)
    ws = torch.empty(max(lib.extend_workspace_bytes(ls, 0, 4, 1), 256), dtype=torch.uint8, device=gpu)
    out = torch.full((0, 2, 128), 7.0, dtype=torch.bfloat16, device=gpu)
    e = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=gpu)
    e1 = torch.empty((0, 1, 128), dtype=torch.bfloat16, device=gpu)
    lib.extend_attn(ls, dc, e, e1, e1, to_dev_i32([0, 0], gpu), to_dev_i32([0], gpu), to_dev_i32(np.zeros((1, 4)), gpu),
                    out, ws, 1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("sink,recent", [(0, 1), (16, 5), (128, 100), (64, 256)])
def test_other_sink_recent_on_poisoned_cache(gpu, sink, recent):
    """Every cache byte starts as 0xFF (NaN in every scale, zero and BF16 row):
    no unwritten slot may reach the output, whatever the region sizes."""
    rng = np.random.default_rng(600 + sink + recent)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8, sink=sink, recent=recent)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    prefix = [0, 9, sink + recent + 3, 333, 700]
    chunks = [4, 20, 2, 16, 31]
    table = synth.permuted_page_table(rng, len(prefix), 50)
    cache = O.new_cache(shape, int(table.max()) + 1, len(prefix))
    for f in ("pages", "k_sink", "v_sink", "k_ring", "v_ring"):
        getattr(cache, f)[...] = np.iinfo(getattr(cache, f).dtype).max
    fill_prefix(shape, cache, layer, law, rng, prefix, table)
    res, *_ = run_extend(gpu, shape, cache, layer, law, rng, prefix, chunks, table)
    print(sink, recent, "poisoned extend", res, flush=True)


def test_chunked_prefill_through_the_library(gpu):
    """A 1,500-token prompt prefilled in chunks of 512, 512, 476 the way a
    serving loop does it: extend over the cache the library wrote so far, then
    kv_write of the chunk.  Each extend is checked against the oracle's extend
    over the same (library-written) cache bytes; the last step also against a
    decode of the written cache, which must see the same keys."""
    import torch
    import int2_rotated_kv_write_amd as lib
    rng = np.random.default_rng(9)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    table = synth.permuted_page_table(rng, 1, 100)
    dc = device_cache(shape, O.new_cache(shape, int(table.max()) + 1, 1), layer, gpu)
    ls = lib_shape(shape)
    table_d = to_dev_i32(table, gpu)
    L = 0
    for n in (512, 512, 476):
        res, q, k, v = run_extend(gpu, shape, host_cache(dc), layer, law, rng, [L], [n], table, dc=dc)
        print("chunk at", L, res, flush=True)
        lib.kv_write(ls, dc, to_dev_bf16(k, gpu), to_dev_bf16(v, gpu), to_dev_i32(np.zeros(n), gpu),
                     to_dev_i32(np.arange(L, L + n), gpu), table_d, to_dev_i32([L + n], gpu))
        L += n
    torch.cuda.synchronize()
    cache = host_cache(dc)
    q = synth.decode_queries(rng, 1, 8)
    want = O.decode(shape, cache, layer, q, table, [L], SIG)
    ws = torch.empty(lib.decode_workspace_bytes(ls, 1, 100), dtype=torch.uint8, device=gpu)
    out = torch.empty((1, 8, 128), dtype=torch.bfloat16, device=gpu)
    lib.decode_attn(ls, dc, to_dev_bf16(q, gpu), table_d, to_dev_i32([L], gpu), out, ws, SIG)
    torch.cuda.synchronize()
    print("decode after prefill", compare_outputs(from_dev_bf16(out), want), flush=True)
