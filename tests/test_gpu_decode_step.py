"""GPU: oscar_decode_step is exactly kv_write followed by decode_attn.

Two identical device caches are prefilled; then several decode steps append
one token per sequence and decode, on one cache through the two separate
calls and on the other through decode_step.  Caches and outputs must be
bit-identical after every step, and the last step's output is held to the
oracle (rules of gpu_harness.py) decoding the same GPU-written cache."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_harness import (SIG, compare_outputs, device_cache, from_dev_bf16, host_cache, lib_shape, to_dev_bf16,
                         to_dev_i32)

pytestmark = pytest.mark.gpu


def _layer(rng, law, G):
    qc, kc, vc = synth.calibration_samples(rng, law, G, 1024)
    cal = O.calibrate_layer(qc, kc, vc, SIG)
    return O.Layer(cal["u_k"], cal["u_v"], cal["clip_k"], cal["clip_v"])


def _same_cache(a: O.Cache, b: O.Cache):
    for f in ("pages", "k_sink", "v_sink", "k_ring", "v_ring"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("H,G,B", [(2, 4, 3), (1, 8, 3), (8, 4, 28)])
def test_decode_step_equals_write_then_decode(gpu, H, G, B):
    """(8, 4, 28) is the benchmark's launch: 28 sequences x 8 KV heads, one new
    token each, G = 4 (the many-pairs plan and the front kernel's flattened
    write grid at that size)."""
    import torch
    import int2_rotated_kv_write_amd as lib
    rng = np.random.default_rng(40 + G + B)
    shape = O.Shape(num_kv_heads=H, num_q_heads=H * G)
    law = synth.outlier_law(rng, H)
    layer = _layer(rng, law, G)
    lens0 = np.array([700, 1301, 2000]) if B == 3 else rng.integers(600, 2100, B)
    steps = 3 if B == 3 else 2
    max_pages = int(np.ceil((lens0.max() + steps) / 16))
    table = synth.permuted_page_table(rng, B, max_pages)
    Lf = lens0 + steps - 1                       # lengths after the last step's write
    kv = [(law.sample_bf16(rng, int(L)), law.sample_bf16(rng, int(L))) for L in Lf]
    ls = lib_shape(shape)
    empty = O.new_cache(shape, B * max_pages, B)
    ca, cb = device_cache(shape, empty, layer, gpu), device_cache(shape, empty, layer, gpu)
    table_d = to_dev_i32(table, gpu)
    # prefill positions [0, L0 - 1) of every sequence, identically in both caches
    for b, L in enumerate(lens0):
        n = int(L) - 1
        args = (to_dev_bf16(kv[b][0][:n], gpu), to_dev_bf16(kv[b][1][:n], gpu), to_dev_i32(np.full(n, b), gpu),
                to_dev_i32(np.arange(n), gpu), table_d, to_dev_i32(lens0 - 1, gpu))
        lib.kv_write(ls, ca, *args)
        lib.kv_write(ls, cb, *args)
    ws_a = torch.empty(lib.decode_workspace_bytes(ls, B, max_pages), dtype=torch.uint8, device=gpu)
    ws_b = torch.empty_like(ws_a)
    idx = to_dev_i32(np.arange(B), gpu)
    for s in range(steps):
        pos = lens0 - 1 + s
        lens = pos + 1
        k_new = to_dev_bf16(np.stack([kv[b][0][pos[b]] for b in range(B)]), gpu)
        v_new = to_dev_bf16(np.stack([kv[b][1][pos[b]] for b in range(B)]), gpu)
        q = to_dev_bf16(synth.decode_queries(rng, B, H * G), gpu)
        pos_d, lens_d = to_dev_i32(pos, gpu), to_dev_i32(lens, gpu)
        out_a = torch.full((B, H * G, 128), float("nan"), dtype=torch.bfloat16, device=gpu)
        out_b = torch.full_like(out_a, float("nan"))
        print(f"decode_step H={H} G={G} step {s}", flush=True)
        lib.kv_write(ls, ca, k_new, v_new, idx, pos_d, table_d, lens_d)
        lib.decode_attn(ls, ca, q, table_d, lens_d, out_a, ws_a, SIG)
        lib.decode_step(ls, cb, k_new, v_new, idx, pos_d, lens_d, q, table_d, lens_d, out_b, ws_b, SIG)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
        _same_cache(host_cache(ca), host_cache(cb))
    # the last step against the oracle decoding the cache the GPU wrote (the decode
    # parity rule: write-side near-tie code differences are checked by the kv_write
    # tests, not folded into the attention output)
    out_ref = O.decode(shape, host_cache(cb), layer, from_dev_bf16(q), table, Lf, SIG)
    print(compare_outputs(from_dev_bf16(out_b), out_ref), flush=True)


def test_decode_step_decode_only_and_write_only(gpu):
    """num_tokens == 0 decodes only; batch == 0 writes only."""
    import torch
    import int2_rotated_kv_write_amd as lib
    rng = np.random.default_rng(7)
    shape = O.Shape(num_kv_heads=1, num_q_heads=4)
    law = synth.outlier_law(rng, 1)
    layer = _layer(rng, law, 4)
    L = 900
    table = synth.contiguous_page_table(1, 64)
    k, v = law.sample_bf16(rng, L), law.sample_bf16(rng, L)
    ref = O.new_cache(shape, 64, 1)
    O.kv_write(shape, ref, layer, k, v, np.zeros(L, int), np.arange(L), table, [L])
    ls = lib_shape(shape)
    dc = device_cache(shape, ref, layer, gpu)
    table_d, lens_d = to_dev_i32(table, gpu), to_dev_i32([L], gpu)
    q = synth.decode_queries(rng, 1, 4)
    ws = torch.empty(lib.decode_workspace_bytes(ls, 1, 64), dtype=torch.uint8, device=gpu)
    out = torch.full((1, 4, 128), float("nan"), dtype=torch.bfloat16, device=gpu)
    none_i = torch.empty(0, dtype=torch.int32, device=gpu)
    lib.decode_step(ls, dc, None, None, none_i, none_i, lens_d, to_dev_bf16(q, gpu), table_d, lens_d, out, ws, SIG)
    torch.cuda.synchronize()
    compare_outputs(from_dev_bf16(out), O.decode(shape, ref, layer, q, table, [L], SIG))
    # write only: a new token at position L on one copy through kv_write, on another
    # through decode_step with batch 0; the caches must match byte for byte
    k1, v1 = law.sample_bf16(rng, 1), law.sample_bf16(rng, 1)
    dc2 = device_cache(shape, ref, layer, gpu)
    dc3 = device_cache(shape, ref, layer, gpu)
    wargs = (to_dev_bf16(k1, gpu), to_dev_bf16(v1, gpu), to_dev_i32([0], gpu), to_dev_i32([L], gpu))
    after = to_dev_i32([L + 1], gpu)
    lib.kv_write(ls, dc2, *wargs, table_d, after)
    lib.decode_step(ls, dc3, *wargs, after, to_dev_bf16(q[:0], gpu), table_d, none_i, out[:0], ws, SIG)
    torch.cuda.synchronize()
    _same_cache(host_cache(dc2), host_cache(dc3))
