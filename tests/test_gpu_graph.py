"""GPU: the library's calls can be captured in a HIP graph.

The library allocates nothing, issues no memset and never synchronises, so
a decode step (decode_step, decode_attn, bf16_decode_attn) captured into a
graph must replay to the eager results.  The graph is replayed three times
with eager work (clearing the outputs, an unrelated kernel) between the
replays; every replay must match the eager call bit for bit.  Re-writing
the same new token at the same position is idempotent, so every replay of
decode_step starts from the same cache."""
import math

import numpy as np
import pytest

import oracle as O
import synth
from gpu_harness import SIG, device_cache, lib_shape, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager(gpu):
    import torch
    import int2_rotated_kv_write_amd as lib
    rng = np.random.default_rng(90)
    H, G = 2, 4
    shape = O.Shape(num_kv_heads=H, num_q_heads=H * G)
    law = synth.outlier_law(rng, H)
    qc, kc, vc = synth.calibration_samples(rng, law, G, 512)
    cal = O.calibrate_layer(qc, kc, vc, SIG)
    layer = O.Layer(cal["u_k"], cal["u_v"], cal["clip_k"], cal["clip_v"])
    lens = np.array([1200, 777])
    B = len(lens)
    max_pages = int(np.ceil(lens.max() / 16))
    table = synth.permuted_page_table(rng, B, max_pages)
    ls = lib_shape(shape)
    cache = device_cache(shape, O.new_cache(shape, B * max_pages, B), layer, gpu)
    table_d = to_dev_i32(table, gpu)
    kv = [(law.sample_bf16(rng, int(L)), law.sample_bf16(rng, int(L))) for L in lens]
    for b, L in enumerate(lens):   # prefill [0, L - 1)
        n = int(L) - 1
        lib.kv_write(ls, cache, to_dev_bf16(kv[b][0][:n], gpu), to_dev_bf16(kv[b][1][:n], gpu),
                     to_dev_i32(np.full(n, b), gpu), to_dev_i32(np.arange(n), gpu), table_d,
                     to_dev_i32(lens - 1, gpu))
    k_new = to_dev_bf16(np.stack([kv[b][0][lens[b] - 1] for b in range(B)]), gpu)
    v_new = to_dev_bf16(np.stack([kv[b][1][lens[b] - 1] for b in range(B)]), gpu)
    idx, pos, lens_d = to_dev_i32(np.arange(B), gpu), to_dev_i32(lens - 1, gpu), to_dev_i32(lens, gpu)
    q = to_dev_bf16(synth.decode_queries(rng, B, H * G), gpu)
    ws = torch.empty(lib.decode_workspace_bytes(ls, B, max_pages), dtype=torch.uint8, device=gpu)
    # BF16 baseline pages of the same tokens (placement by the oracle's writer)
    b16 = O.new_bf16_pages(B * max_pages, H)
    for b, L in enumerate(lens):
        O.bf16_pages_write(b16, kv[b][0], kv[b][1], np.full(int(L), b), np.arange(int(L)), table)
    b16_d = to_dev_bf16(b16, gpu)
    ws16 = torch.empty(lib.bf16_decode_workspace_bytes(H, H * G, B, max_pages), dtype=torch.uint8, device=gpu)

    outs = [torch.empty((B, H * G, 128), dtype=torch.bfloat16, device=gpu) for _ in range(3)]

    def calls():
        lib.decode_step(ls, cache, k_new, v_new, idx, pos, lens_d, q, table_d, lens_d, outs[0], ws, SIG)
        lib.decode_attn(ls, cache, q, table_d, lens_d, outs[1], ws, SIG)
        lib.bf16_decode_attn(H, H * G, b16_d, q, table_d, lens_d, outs[2], ws16, SIG)

    calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()   # warm up on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.randn(1 << 20, device=gpu).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("decode_step", "decode_attn", "bf16_decode_attn"), outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), (rep, name)
    print("graph replays match eager", flush=True)
