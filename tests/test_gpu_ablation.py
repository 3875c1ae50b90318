"""Rotation ablation through the library's kernels: the Hadamard-only rotation
(U = I) and the naive INT2 baseline (U = bf16(P H), so R = U H P ~ I) are only
other U inputs to kv_write and decode_attn.  Parity of those paths with the
oracle, and the ordering the Spanish summary's section 4 and the Italian page's
"Analisi delle Prestazioni" report: naive INT2 collapses, with an
attention-output error several times that of either rotated variant."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle as O
import synth
from gpu_harness import SIG, device_cache, from_dev_bf16, lib_shape, to_dev_bf16, to_dev_i32
from test_gpu_parity import run_scenario

pytestmark = pytest.mark.gpu


def fixed_basis_layer(kc, vc, basis, H):
    """Layer with U_K = U_V = bf16(basis) per head and the oracle-side clip quantile."""
    u = O.f64_to_bf16(np.broadcast_to(basis, (H, 128, 128)))
    clip = lambda x: np.float32(np.quantile(np.concatenate([np.abs(x[h] @ O.rotation(u[h])).ravel()
                                                           for h in range(H)]), 0.999))
    return O.Layer(u, u.copy(), clip(kc), clip(vc))


def naive_basis():
    return O.bitrev_permutation() @ O.hadamard()


@pytest.mark.parametrize("basis", ["identity", "naive"])
def test_write_and_decode_parity_with_a_fixed_basis(gpu, basis):
    """kv_write + decode_attn with U = I or U = bf16(P H) match the oracle under
    the usual parity rules (the kernels take any bf16 U)."""
    rng = np.random.default_rng(31 if basis == "identity" else 32)
    shape = O.Shape(num_kv_heads=2, num_q_heads=8)
    law = synth.outlier_law(rng, 2)
    _, kc, vc = synth.calibration_samples(rng, law, 4, 256)
    layer = fixed_basis_layer(kc, vc, np.eye(128) if basis == "identity" else naive_basis(), 2)
    lens = [1000, 333]
    table = synth.permuted_page_table(rng, 2, 70)
    calls = [(np.full(L, s), np.arange(L)) for s, L in enumerate(lens)]
    stats, res = run_scenario(gpu, shape, layer, law, lens, table, calls, rng)
    print(basis, "decode", res, flush=True)


def test_naive_int2_collapses_and_rotations_do_not(gpu):
    """Attention-output error against exact attention over the bf16 K/V, through
    the kernels, on the outlier law with rank-8 queries that avoid the outlier
    channels: naive INT2 is at least three times worse than either rotation."""
    import torch
    import int2_rotated_kv_write_amd as lib
    rng = np.random.default_rng(33)
    shape = O.Shape(num_kv_heads=1, num_q_heads=4)
    law = synth.outlier_law(rng, 1)
    q_law = synth.lowrank_query_law(rng, law, 8)
    qc, kc, vc = synth.calibration_samples(rng, law, 4, 2048, q_law)
    cal = O.calibrate_layer(qc, kc, vc, SIG)
    layers = {"oscar": O.Layer(cal["u_k"], cal["u_v"], cal["clip_k"], cal["clip_v"]),
              "hadamard_only": fixed_basis_layer(kc, vc, np.eye(128), 1),
              "naive_int2": fixed_basis_layer(kc, vc, naive_basis(), 1)}
    B, L = 4, 2048
    table = synth.contiguous_page_table(B, L // 16)
    k = np.stack([law.sample_bf16(rng, L) for _ in range(B)])       # [B][L][1][128]
    v = np.stack([law.sample_bf16(rng, L) for _ in range(B)])
    q = q_law.decode_queries(rng, B, 4)
    ref = np.zeros((B, 4, 128))
    for b in range(B):
        K, V = O.bf16_to_f64(k[b, :, 0]), O.bf16_to_f64(v[b, :, 0])
        for hq in range(4):
            lg = SIG * (K @ O.bf16_to_f64(q[b, hq]))
            p = np.exp(lg - lg.max())
            ref[b, hq] = (p @ V) / p.sum()
    seq = np.repeat(np.arange(B), L)
    pos = np.tile(np.arange(L), B)
    ls = lib_shape(shape)
    err = {}
    for name, layer in layers.items():
        dc = device_cache(shape, O.new_cache(shape, B * L // 16, B), layer, gpu)
        lib.kv_write(ls, dc, to_dev_bf16(k.reshape(B * L, 1, 128), gpu), to_dev_bf16(v.reshape(B * L, 1, 128), gpu),
                     to_dev_i32(seq, gpu), to_dev_i32(pos, gpu), to_dev_i32(table, gpu), to_dev_i32([L] * B, gpu))
        out = torch.empty((B, 4, 128), dtype=torch.bfloat16, device=gpu)
        ws = torch.empty(lib.decode_workspace_bytes(ls, B, L // 16), dtype=torch.uint8, device=gpu)
        lib.decode_attn(ls, dc, to_dev_bf16(q, gpu), to_dev_i32(table, gpu), to_dev_i32([L] * B, gpu), out, ws, SIG)
        torch.cuda.synchronize()
        got = O.bf16_to_f64(from_dev_bf16(out))
        err[name] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print("relative output error", err, flush=True)
    # i.i.d. synthetic K/V give nearly flat attention over 2,048 keys, whose output is
    # small next to the INT2 error: the relative errors exceed 1 for every variant,
    # and only their ratio is the finding
    assert all(math.isfinite(e) for e in err.values())
    assert err["naive_int2"] >= 3 * err["oscar"]
    assert err["naive_int2"] >= 3 * err["hadamard_only"]
