"""GPU parity of cascade decode (decode_attn_cascade) against the oracle's
decode: groups of sequences whose page tables name the same physical pages for
a common prefix (a prefix-cache hit: the Spanish summary, 2.2 B and section 3,
item 3; the Italian page's section "Architettura del Sistema di Serving e
Layout di Memoria") have those pages read once per block of query heads.  The
result is decode attention over each sequence's own cache view, so the oracle
is decode itself; outputs are held to the decode tolerance (gpu_harness)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import synth
from gpu_harness import SIG, compare_outputs, device_cache, from_dev_bf16, lib_shape, to_dev_bf16, to_dev_i32
from test_gpu_parity import make_layer

pytestmark = pytest.mark.gpu


def shared_cache(shape, layer, law, rng, lens, groups, max_pages, poison=False):
    """Oracle cache in which the members of each group (b0, b1, prefix_tokens) share
    the physical pages of their first prefix_tokens tokens and hold the same token
    values there; every other page is private.  Returns (cache, table)."""
    B = len(lens)
    H = shape.num_kv_heads
    need = [-(-L // 16) for L in lens]
    owner_pages = {}
    table = np.zeros((B, max_pages), np.int32)
    nxt = 0
    perm = rng.permutation(sum(need) + 1).astype(np.int32)
    group_of = {}
    for gi, (b0, b1, pt) in enumerate(groups):
        for b in range(b0, b1):
            group_of[b] = (gi, pt // 16)
    for b in range(B):
        gi, pp = group_of.get(b, (None, 0))
        for j in range(need[b]):
            if gi is not None and j < pp and (gi, j) in owner_pages:
                table[b, j] = owner_pages[(gi, j)]
            else:
                table[b, j] = perm[nxt]
                nxt += 1
                if gi is not None and j < pp:
                    owner_pages[(gi, j)] = table[b, j]
    cache = O.new_cache(shape, int(table.max()) + 1, B)
    if poison:
        for f in ("pages", "k_sink", "v_sink", "k_ring", "v_ring"):
            getattr(cache, f)[...] = np.iinfo(getattr(cache, f).dtype).max
    prefix = {}
    for b in range(B):
        k, v = law.sample_bf16(rng, lens[b]), law.sample_bf16(rng, lens[b])
        if b in group_of:
            gi, pp = group_of[b]
            n = min(16 * pp, lens[b])
            if gi not in prefix:
                prefix[gi] = (law.sample_bf16(rng, 16 * pp), law.sample_bf16(rng, 16 * pp))
            k[:n], v[:n] = prefix[gi][0][:n], prefix[gi][1][:n]
        O.kv_write(shape, cache, layer, k, v, np.full(lens[b], b), np.arange(lens[b]), table, lens)
    assert H >= 1
    return cache, table


def run_cascade(device, shape, cache, layer, table, lens, cu_groups, group_pages, max_group, max_shared, rng):
    import torch
    import int2_rotated_kv_write_amd as lib
    B = len(lens)
    ls = lib_shape(shape)
    q = synth.decode_queries(rng, B, shape.num_q_heads)
    want = O.decode(shape, cache, layer, q, table, lens, SIG)
    dc = device_cache(shape, cache, layer, device)
    ws = torch.empty(lib.cascade_workspace_bytes(ls, B, table.shape[1], max_shared), dtype=torch.uint8, device=device)
    ws.fill_(0xFF)
    out = torch.full((B, shape.num_q_heads, 128), float("nan"), dtype=torch.bfloat16, device=device)
    q_d, table_d, lens_d = to_dev_bf16(q, device), to_dev_i32(table, device), to_dev_i32(lens, device)
    lib.decode_attn_cascade(ls, dc, q_d, table_d, lens_d, to_dev_i32(cu_groups, device),
                            to_dev_i32(group_pages, device), out, ws, max_group, max_shared, SIG)
    torch.cuda.synchronize()
    res = compare_outputs(from_dev_bf16(out), want)
    # the same call without sharing: decode_attn over the same cache
    ws2 = torch.empty(lib.decode_workspace_bytes(ls, B, table.shape[1]), dtype=torch.uint8, device=device)
    out2 = torch.empty_like(out)
    lib.decode_attn(ls, dc, q_d, table_d, lens_d, out2, ws2, SIG)
    torch.cuda.synchronize()
    d = (out.float() - out2.float()).abs().max().item()
    return res, d


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_two_groups_and_loners(gpu, G):
    """Six sequences: a group of three sharing 1,664 tokens (100 INT2 pages), one
    of them too short to hold every shared page inside its INT2 history (it reads
    its pages itself); a group of two sharing 64 + 16 * 37 tokens; one sequence in
    no group."""
    rng = np.random.default_rng(70 + G)
    shape = O.Shape(num_kv_heads=2, num_q_heads=2 * G)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [3001, 2500, 1800, 1200, 900, 2049]
    groups = [(0, 3, 64 + 16 * 100), (3, 5, 64 + 16 * 37)]
    cache, table = shared_cache(shape, layer, law, rng, lens, groups, 200)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0, 3, 5], [100, 37], 3, 100, rng)
    print("G", G, "cascade", res, "vs decode_attn", d, flush=True)


@pytest.mark.parametrize("G", [4, 8])
def test_shared_prefix_over_many_ranges(gpu, G):
    """A group of five sharing 4,160 tokens (256 INT2 pages): with few
    (sequence, KV head) pairs the plan's ranges are short, so the shared prefix
    spans many shared ranges; a sixth sequence shares nothing."""
    rng = np.random.default_rng(80 + G)
    shape = O.Shape(num_kv_heads=1, num_q_heads=G)
    law = synth.outlier_law(rng, 1)
    layer = make_layer(rng, shape, law, 256)
    lens = [4700, 6000, 4500, 5123, 4416, 3000]
    groups = [(0, 5, 64 + 16 * 256)]
    cache, table = shared_cache(shape, layer, law, rng, lens, groups, 400)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0, 5], [256], 5, 256, rng)
    print("G", G, "long shared prefix", res, "vs decode_attn", d, flush=True)


def test_max_group_below_group_size(gpu):
    """max_group 2 with a group of four: the first two members use the shared
    reads, the others read their pages themselves."""
    rng = np.random.default_rng(90)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [2000, 2100, 2200, 2300]
    groups = [(0, 4, 64 + 16 * 90)]
    cache, table = shared_cache(shape, layer, law, rng, lens, groups, 160)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0, 4], [90], 2, 90, rng)
    print("max_group 2", res, d, flush=True)


def test_no_groups_equals_decode(gpu):
    rng = np.random.default_rng(91)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [700, 1500]
    cache, table = shared_cache(shape, layer, law, rng, lens, [], 120)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0], np.zeros(0, np.int32), 1, 50, rng)
    assert d == 0.0, "without groups the cascade call is decode_attn"


@pytest.mark.parametrize("sink,recent", [(0, 1), (16, 5), (64, 256)])
def test_poisoned_cache_with_sharing(gpu, sink, recent):
    """Every cache byte starts as 0xFF; a group of three shares 50 INT2 pages
    (one member's INT2 history ends inside them)."""
    rng = np.random.default_rng(95 + sink + recent)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8, sink=sink, recent=recent)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [sink + 16 * 50 + recent + 40, sink + 16 * 50 + recent + 3, sink + 16 * 30, 500]
    groups = [(0, 3, sink + 16 * 50)]
    cache, table = shared_cache(shape, layer, law, rng, lens, groups, 80, poison=True)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0, 3], [50], 3, 50, rng)
    print(sink, recent, "poisoned cascade", res, d, flush=True)


def test_ragged_batch_with_a_quarter_sharing(gpu):
    """The ragged serving mix at reduced size: 16 sequences of 4K to 12K tokens,
    64 query / 8 KV heads cut to 16 / 2, the first quarter sharing a 4,096-token
    prefix."""
    rng = np.random.default_rng(99)
    shape = O.Shape(num_kv_heads=2, num_q_heads=16)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [int(x) for x in rng.integers(4200, 12000, size=16)]
    groups = [(0, 4, 4096)]
    cache, table = shared_cache(shape, layer, law, rng, lens, groups, 750)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0, 4], [(4096 - 64) // 16], 4, 252, rng)
    print("ragged 16 with sharing", res, d, flush=True)


def test_short_first_member_shares_nothing(gpu):
    """The first member's INT2 history ends inside the shared pages: the shared
    pages are read through its page-table row, so the whole group reads its
    pages itself (the result is still decode's)."""
    rng = np.random.default_rng(97)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    law = synth.outlier_law(rng, 2)
    layer = make_layer(rng, shape, law, 256)
    lens = [64 + 16 * 60, 64 + 16 * 80 + 300, 64 + 16 * 80 + 999]
    groups = [(0, 3, 64 + 16 * 80)]
    cache, table = shared_cache(shape, layer, law, rng, lens, groups, 160)
    res, d = run_cascade(gpu, shape, cache, layer, table, lens, [0, 3], [80], 3, 80, rng)
    print("short first member", res, d, flush=True)
