"""GPU: oscar_decode_attn_noalloc (static library scratch, no workspace) gives
the same outputs as oscar_decode_attn with a caller workspace, bit for bit,
on two calls in a row, the second with a smaller batch and shorter sequences
(the scratch keeps the first call's contents), and both stay within the
oracle's tolerance."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_harness import SIG, compare_outputs, device_cache, from_dev_bf16, lib_shape, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


def _case(rng, shape, law, layer, lens, max_pages):
    table = synth.permuted_page_table(rng, len(lens), max_pages)
    ref = O.new_cache(shape, int(table.max()) + 1, len(lens))
    for b, L in enumerate(lens):
        O.kv_write(shape, ref, layer, law.sample_bf16(rng, L), law.sample_bf16(rng, L), np.full(L, b),
                   np.arange(L), table, lens)
    q = synth.decode_queries(rng, len(lens), shape.num_q_heads)
    return table, ref, q


def test_noalloc_matches_workspace_decode_twice(gpu):
    import torch
    import int2_rotated_kv_write_amd as lib
    rng = np.random.default_rng(901)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    law = synth.outlier_law(rng, 2)
    qc, kc, vc = synth.calibration_samples(rng, law, shape.gqa, 256)
    cal = O.calibrate_layer(qc, kc, vc, SIG)
    layer = O.Layer(cal["u_k"], cal["u_v"], cal["clip_k"], cal["clip_v"])
    ls = lib_shape(shape)
    for call, (lens, max_pages) in enumerate((([2049, 700, 321, 65, 1], 130), ([900, 17], 60))):
        print(f"noalloc call {call}: lens {lens}", flush=True)
        table, ref, q = _case(rng, shape, law, layer, lens, max_pages)
        dc = device_cache(shape, ref, layer, gpu)
        B = len(lens)
        q_d, t_d, l_d = to_dev_bf16(q, gpu), to_dev_i32(table, gpu), to_dev_i32(lens, gpu)
        ws = torch.empty(lib.decode_workspace_bytes(ls, B, max_pages), dtype=torch.uint8, device=gpu)
        out_ws = torch.full((B, shape.num_q_heads, 128), float("nan"), dtype=torch.bfloat16, device=gpu)
        out_na = torch.full_like(out_ws, float("nan"))
        lib.decode_attn(ls, dc, q_d, t_d, l_d, out_ws, ws, SIG)
        lib.decode_attn_noalloc(ls, dc, q_d, t_d, l_d, out_na, SIG)
        torch.cuda.synchronize()
        assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16)), f"call {call}"
        res = compare_outputs(from_dev_bf16(out_na), O.decode(shape, ref, layer, q, table, lens, SIG))
        print(f"noalloc call {call}: bit-identical to decode_attn, oracle {res}", flush=True)


def test_noalloc_rejects_oversize_batch(gpu):
    """A batch whose scratch need exceeds the static array is an argument error,
    raised before any launch."""
    import torch
    import int2_rotated_kv_write_amd as lib
    shape = O.Shape(num_kv_heads=8, num_q_heads=32)
    ls = lib_shape(shape)
    top = 4 + 1023 * 512
    assert lib.decode_workspace_bytes(ls, 64, top) > lib._native.NOALLOC_SCRATCH_BYTES
    layer = O.Layer(np.zeros((8, 128, 128), np.uint16), np.zeros((8, 128, 128), np.uint16),
                    np.float32(1), np.float32(1))
    dc = device_cache(shape, O.new_cache(shape, 1, 64), layer, gpu)
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=gpu)
    out = torch.empty_like(q)
    table = torch.zeros((64, top), dtype=torch.int32, device=gpu)
    lens = torch.zeros(64, dtype=torch.int32, device=gpu)
    with pytest.raises(lib.OscarError, match="OSCAR_NOALLOC_SCRATCH_BYTES"):
        lib.decode_attn_noalloc(ls, dc, q, table, lens, out, SIG)
