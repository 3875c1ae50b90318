"""GPU parity of the BF16 paged decode (the baseline the pages measure OSCAR
against) with the oracle's decode_bf16_paged, rules of gpu_harness.py.

Small cases fill the pages with the oracle's writer and poison every slot
past each sequence's end with NaN bit patterns, so any unmasked read shows.
The full-size case is one layer of the benchmark's 28 x 100,000-token
workload in the launch the benchmark times; sampled (sequence, KV head)
pairs are re-derived by the oracle from their downloaded pages."""
import math

import numpy as np
import pytest

import oracle as O
import synth
from gpu_harness import SIG, compare_outputs, from_dev_bf16, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC1


def run_case(device, H, G, lens, seed, table_kind="permuted", law_kind="outlier"):
    import torch
    import int2_rotated_kv_write_amd as lib
    rng = np.random.default_rng(seed)
    B, Hq = len(lens), H * G
    max_pages = max(1, max(math.ceil(L / 16) for L in lens))
    table = synth.permuted_page_table(rng, B, max_pages) if table_kind == "permuted" \
        else synth.contiguous_page_table(B, max_pages)
    pages = np.full((B * max_pages, H, O.BF16_BLOCK), NAN_BF16, np.uint16)
    law = synth.outlier_law(rng, H) if law_kind == "outlier" else synth.heavy_tail_law(rng, H)
    for b, L in enumerate(lens):
        if L:
            O.bf16_pages_write(pages, law.sample_bf16(rng, L), law.sample_bf16(rng, L),
                               np.full(L, b), np.arange(L), table)
    q = synth.decode_queries(rng, B, Hq)
    ref = O.decode_bf16_paged(pages, q, table, lens, H, SIG)
    pages_d = to_dev_bf16(pages, device)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.bfloat16, device=device)
    ws = torch.empty(lib.bf16_decode_workspace_bytes(H, Hq, B, max_pages), dtype=torch.uint8, device=device)
    print(f"bf16 decode: H={H} G={G} lens={lens} seed={seed}", flush=True)
    lib.bf16_decode_attn(H, Hq, pages_d, to_dev_bf16(q, device), to_dev_i32(table, device),
                         to_dev_i32(lens, device), out, ws, SIG)
    torch.cuda.synchronize()
    return compare_outputs(from_dev_bf16(out), ref)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_ragged_lengths_permuted_pages(gpu, G):
    """Lengths around page boundaries and across many ranges per (sequence,
    KV head): 1, 15, 16, 17, 100, 1000, 5003 tokens."""
    stats = run_case(gpu, 2, G, [1, 15, 16, 17, 100, 1000, 5003], seed=G)
    print(stats)


def test_tiny_gqa4_1k(gpu):
    stats = run_case(gpu, 1, 4, [1024], seed=0, table_kind="contiguous")
    print(stats)


def test_zero_lengths_and_heavy_law(gpu):
    stats = run_case(gpu, 8, 4, [0, 3000, 0, 64], seed=11, law_kind="heavy")
    print(stats)


def test_concurrent_28x100k_sampled(gpu):
    """28 sequences x 100,000 tokens, 32 query / 8 KV heads, permuted pages,
    heavy law, one call as the benchmark times it; 4 sampled (sequence, KV
    head) pairs re-derived by the oracle."""
    import torch
    import int2_rotated_kv_write_amd as lib
    from synth.device import fill_bf16_pages_device, sample_kv_device, sample_queries_device
    H, Hq, B, L = 8, 32, 28, 100_000
    rng = np.random.default_rng(0)
    law = synth.heavy_tail_law(rng, H)
    P = math.ceil(L / 16)
    table = synth.permuted_page_table(rng, B, P)
    table_d = to_dev_i32(table, gpu)
    pages = torch.empty((B * P, H, O.BF16_BLOCK), dtype=torch.bfloat16, device=gpu)
    gen = torch.Generator(device=gpu)
    gen.manual_seed(0)
    for b in range(B):
        fill_bf16_pages_device(pages, sample_kv_device(law, L, gen, gpu), sample_kv_device(law, L, gen, gpu),
                               table_d[b])
    q = sample_queries_device(B, Hq, gen, gpu)
    lens = [L] * B
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=gpu)
    ws = torch.empty(lib.bf16_decode_workspace_bytes(H, Hq, B, P), dtype=torch.uint8, device=gpu)
    print("bf16 decode 28 x 100K: launching", flush=True)
    lib.bf16_decode_attn(H, Hq, pages, q, table_d, to_dev_i32(lens, gpu), out, ws, SIG)
    torch.cuda.synchronize()
    got = from_dev_bf16(out)
    q_h = from_dev_bf16(q)
    for b, h in ((0, 0), (13, 5), (27, 7), (6, 2)):
        blocks = from_dev_bf16(pages[table_d[b].long(), h:h + 1])   # [P][1][4096]
        ref = O.decode_bf16_paged(blocks, q_h[b:b + 1, h * 4:(h + 1) * 4], np.arange(P, dtype=np.int32)[None],
                                  [L], 1, SIG)
        stats = compare_outputs(got[b:b + 1, h * 4:(h + 1) * 4], ref)
        print((b, h), stats, flush=True)
