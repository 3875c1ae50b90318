"""Benchmark: OSCAR INT2 decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (concurrent_28x100k_36l): 28 sequences of 100,000 tokens,
32 query / 8 KV heads, head_dim 128, 36 layers, random permuted page tables
(page 16), sinks 64 + recent 256 in BF16, the rest INT2.  One step = for each
of the 36 layers: kv_write of each sequence's new token (position 99,999),
then decode_attn over the 100,000 cached tokens.  value = decoded tokens/s
(28 per step); each layer's write and decode go through one decode_step
call.  Inputs are seeded synthetic data already resident in HBM.

Besides the headline line's fields, the JSON carries (unless --no-extras):
  single_1x100k     one Qwen3-8B-shaped layer, batch 1, 100,000 tokens,
                    decode_attn over 8 cycled cache copies (HBM-resident);
  ragged_64x4k_128k 64 sequences of 4,096..131,072 tokens, 64 q / 8 kv
                    heads, a quarter of them sharing a 4,096-token prefix:
                    decode_attn and decode_attn_cascade, with the page bytes
                    the shared reads save;
  kv_write_prefill  one kv_write of 100,000 prefill tokens x 8 KV heads;
  bf16_baseline     the all-BF16 paged decode at the headline shape;
  concurrent_28x100k_group128  decode_attn at the headline shape and a 100K
                    prefill kv_write in the 2.25-bit format (one 128-channel
                    group per token);
  extend_1x100k_chunk1024  extend_attn (chunked prefill): 1,024 new tokens
                    of one sequence over its cached 100,000-token prefix and
                    causally over themselves, as attention TFLOP/s;
  rotation_ablation attention-output error against BF16 of OSCAR,
                    Hadamard-only and naive INT2 rotations through the
                    library's kernels on two synthetic laws.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/sec + achieved HBM GB/s (% of peak), 100K ctx, 1 MI355X"
PEAK_HBM_GBS = 8000.0
SIG = 1.0 / math.sqrt(128)

WORKLOADS = {
    "concurrent_28x100k_36l": dict(batch=28, seq_len=100_000, q_heads=32, kv_heads=8, layers=36,
                                   table="permuted", law="heavy"),
    # one layer's shape; 8 copies of its cache (525 MB, twice the 256 MB MALL) are cycled
    # through, so every call reads its pages from HBM
    "qwen3_8b_layer_100k": dict(batch=1, seq_len=100_000, q_heads=32, kv_heads=8, layers=8,
                                table="contiguous", law="heavy"),
    "ragged_64x4k_128k": dict(batch=64, seq_len=(4096, 131072), q_heads=64, kv_heads=8, layers=1,
                              table="shared_prefix", law="outlier"),
    # the headline shape in the 2.25-bit format (one 128-channel group per token), its 36
    # layers cycled exactly as the headline's
    "concurrent_28x100k_group128": dict(batch=28, seq_len=100_000, q_heads=32, kv_heads=8, layers=36,
                                        table="permuted", law="heavy", group=128),
    # chunked prefill: the cached 100,000-token prefix of one sequence, then one chunk of
    # EXTEND_CHUNK new tokens through extend_attn
    "extend_1x100k_chunk1024": dict(batch=1, seq_len=100_000, q_heads=32, kv_heads=8, layers=1,
                                    table="permuted", law="heavy"),
}
EXTEND_CHUNK = 1024
PEAK_F16_MFMA_TFLOPS = 2500.0   # dense fp16 MFMA peak of one MI355X
SHARED_PREFIX_TOKENS = 4096     # ragged workload: 25% of the sequences share their first 4,096 tokens
SINK, RECENT = 64, 256
PREFILL_TOKENS = 100_000        # write-path workload: one kv_write of 100,000 prefill tokens x 8 KV heads


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def int2_tokens(L, sink=64, recent=256):
    return max(sink, L - recent) - sink if L > sink else 0


def bf16_tokens(L, sink=64, recent=256):
    return L if L <= sink else sink + (L - max(sink, L - recent))


def decode_bytes(lens, H, Hq, group=64):
    """Algorithmic HBM bytes of one decode_attn call: 80 B per INT2 token-head
    (72 B with one 128-channel group per token), 512 B per BF16 token-head, q
    and out, one page-table entry per INT2 page, U_K and U_V."""
    per_int2 = 72 if group == 128 else 80
    tot = 0
    for L in lens:
        ni = int2_tokens(int(L))
        tot += H * (ni * per_int2 + bf16_tokens(int(L)) * 512)
        tot += 4 * (math.ceil((64 + ni) / 16) - 4)
    tot += len(lens) * Hq * 128 * 2 * 2
    tot += 2 * H * 128 * 128 * 2
    return tot


def bf16_decode_bytes(lens, H, Hq):
    """Algorithmic HBM bytes of one bf16_decode_attn call: 512 B per token-head
    (K and V), q and out, one page-table entry per page."""
    tot = 0
    for L in lens:
        tot += H * int(L) * 512 + 4 * math.ceil(int(L) / 16)
    return tot + len(lens) * Hq * 128 * 2 * 2


def write_bytes(n_tokens, H, group=64):
    """kv_write of n decode tokens (K and V): read 2x256 B per token-head,
    write 80 B INT2 (72 B with 128-channel groups) + 2x256 B ring copy per
    token-head, U_K and U_V."""
    return n_tokens * H * (512 + (72 if group == 128 else 80) + 512) + 2 * H * 128 * 128 * 2


def prefill_write_bytes(n_tokens, H, sink=64, group=64):
    """kv_write of positions [0, n) of one sequence (K and V): read 2x256 B
    per token-head, write 80 B INT2 (72 B with 128-channel groups) per
    token-head at pos >= sink and 2x256 B BF16 per sink or recent token-head,
    U_K and U_V."""
    per_int2 = 72 if group == 128 else 80
    return (H * (n_tokens * 512 + max(0, n_tokens - sink) * per_int2 + bf16_tokens(n_tokens) * 512)
            + 2 * H * 128 * 128 * 2)


DECODE_SOURCES = ("decode.hip", "common.h", "kernels.h")


def decode_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, "int2_rotated_kv_write_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def read_traffic():
    """Measured HBM bytes per decode_attn call from the committed counter
    summary, valid only for the decode sources it was taken on (else None)."""
    path = os.path.join(ROOT, "profiles", "decode_attn_counters_concurrent_28x100k_36l.md")
    if not os.path.exists(path):
        return None
    sha = decode_source_sha256()
    rec = {}
    for line in open(path):
        if line.startswith("traffic:"):
            for kv in line[len("traffic:"):].split():
                key, val = kv.split("=")
                rec[key] = val
    if rec.get("decode_source_sha256") != sha:
        return None
    return float(rec["bytes_per_call"])


def cpu_baseline(H, layers, seq_len, budget_s=20.0):
    """The fp64 oracle's decode, timed on this host on a bounded sample: one
    sequence x one KV head (4 query heads) at the full length; extrapolated to
    the whole step (batch x KV heads x layers units)."""
    import oracle as O
    import synth
    from threadpoolctl import threadpool_info, threadpool_limits
    rng = np.random.default_rng(1234)
    shape = O.Shape(num_kv_heads=1, num_q_heads=4)
    law = synth.heavy_tail_law(rng, 1)
    qc, kc, vc = synth.calibration_samples(rng, law, 4, 256)
    cal = O.calibrate_layer(qc, kc, vc, SIG)
    layer = O.Layer(cal["u_k"], cal["u_v"], cal["clip_k"], cal["clip_v"])
    pages = math.ceil(seq_len / 16)
    table = synth.contiguous_page_table(1, pages)
    cache = O.new_cache(shape, pages, 1)
    k = law.sample_bf16(rng, seq_len)
    v = law.sample_bf16(rng, seq_len)
    O.kv_write(shape, cache, layer, k, v, np.zeros(seq_len, int), np.arange(seq_len), table, [seq_len])
    q = synth.decode_queries(rng, 1, 4)

    def timed(budget):
        times = []
        t_start = time.perf_counter()
        while len(times) < 3 or (time.perf_counter() - t_start < budget and len(times) < 50):
            t0 = time.perf_counter()
            O.decode(shape, cache, layer, q, table, [seq_len], SIG)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > 3 * budget:
                break
        return statistics.median(times), len(times)

    t_unit, reps = timed(budget_s)
    threads = sum(int(i.get("num_threads", 0)) for i in threadpool_info() if i.get("user_api") == "blas")
    with threadpool_limits(1):
        t_one, reps_one = timed(budget_s / 2)
    return t_unit, reps, max(threads, 1), t_one, reps_one


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None



def build_workload(name, rng, gen, dev, n_fill_minus=0):
    """Sequences, page tables and per-layer caches of a named workload, prefilled
    through kv_write with positions [0, L - n_fill_minus) of every sequence
    (seeded synthetic K/V drawn on the device).  Ragged workloads share the
    first SHARED_PREFIX_TOKENS tokens (same values, same physical pages) among a
    contiguous quarter of the batch."""
    import torch
    from types import SimpleNamespace

    import int2_rotated_kv_write_amd as lib
    import synth
    from synth.device import sample_kv_device
    wl = WORKLOADS[name]
    B, Hq, H, NL = wl["batch"], wl["q_heads"], wl["kv_heads"], wl["layers"]
    if isinstance(wl["seq_len"], tuple):
        lens = synth.ragged_lengths(rng, B, *wl["seq_len"])
    else:
        lens = np.full(B, wl["seq_len"], np.int32)
    max_pages = int(math.ceil(lens.max() / 16))
    shape = lib.CacheShape(H, Hq, group=wl.get("group", 64))
    law = synth.heavy_tail_law(rng, H) if wl["law"] == "heavy" else synth.outlier_law(rng, H)

    # ---- offline calibration (host, native library), one set replicated per layer ----
    t0 = time.perf_counter()
    qc, kc, vc = synth.calibration_samples(rng, law, Hq // H, 2048)
    u_k, u_v, ck, cv = lib.calibrate_layer(qc, kc, vc, SIG, 0.999)
    log(f"{name}: calibration {time.perf_counter() - t0:.1f}s clip_k={ck:.3f} clip_v={cv:.3f}")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    u_k_d, u_v_d = bf(u_k), bf(u_v)

    # ---- page table (shared by the layers' separate cache pools) ----
    sharers = []
    if wl["table"] == "permuted":
        table = synth.permuted_page_table(rng, B, max_pages)
    elif wl["table"] == "shared_prefix":
        n_share = B // 4
        s0 = int(rng.integers(0, B - n_share + 1))
        sharers = list(range(s0, s0 + n_share))
        table, _, _ = synth.shared_prefix_page_table(rng, lens, max_pages, SHARED_PREFIX_TOKENS, sharers)
    else:
        table = synth.contiguous_page_table(B, max_pages)
    num_pages = int(table.max()) + 1
    table_d = torch.from_numpy(table).to(dev)

    # ---- caches ----
    caches = []
    t0 = time.perf_counter()
    after = torch.from_numpy(np.maximum(lens - n_fill_minus, 0).astype(np.int32)).to(dev)
    for layer in range(NL):
        c = lib.allocate_cache(shape, num_pages, B, dev, u_k=u_k_d.clone(), u_v=u_v_d.clone(),
                               clip_k=float(ck), clip_v=float(cv))
        prefix_kv = None
        for b in range(B):
            n = int(lens[b]) - n_fill_minus
            for s0 in range(0, n, 1 << 16):
                m = min(1 << 16, n - s0)
                k = sample_kv_device(law, m, gen, dev)
                v = sample_kv_device(law, m, gen, dev)
                if s0 == 0 and b in sharers:   # shared prefix: same tokens, same physical pages
                    if prefix_kv is None:
                        prefix_kv = (k[:SHARED_PREFIX_TOKENS].clone(), v[:SHARED_PREFIX_TOKENS].clone())
                    k[:SHARED_PREFIX_TOKENS] = prefix_kv[0]
                    v[:SHARED_PREFIX_TOKENS] = prefix_kv[1]
                idx = torch.full((m,), b, dtype=torch.int32, device=dev)
                pos = torch.arange(s0, s0 + m, dtype=torch.int32, device=dev)
                lib.kv_write(shape, c, k, v, idx, pos, table_d, after)
        caches.append(c)
        if layer % 6 == 5 or layer == NL - 1:
            torch.cuda.synchronize()
            log(f"{name}: prefilled {layer + 1}/{NL} layers ({time.perf_counter() - t0:.1f}s)")
    return SimpleNamespace(B=B, Hq=Hq, H=H, NL=NL, lens=lens, max_pages=max_pages, shape=shape, law=law,
                           table=table, table_d=table_d, num_pages=num_pages, caches=caches, sharers=sharers)


def event_us(calls, reps):
    """Mean and median device time (us) of `reps` calls cycled over `calls`, each
    bracketed by HIP events on the stream the library launches on (torch's
    current stream), after one untimed pass over `calls`."""
    import torch
    for c in calls:
        c()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        calls[i % len(calls)]()
        e1.record()
    torch.cuda.synchronize()
    t = [1e3 * e0.elapsed_time(e1) for e0, e1 in ev]
    return statistics.mean(t), statistics.median(t)


def shared_pages_saved(lens, sharers, H, G):
    """INT2 page blocks (1,280 B per page and KV head) that cascade decode does
    not read on the ragged workload: every sharer whose INT2 history holds the
    shared pages whole takes them from one read per block of 16 ceil(G / 4) of
    the sharers' query heads instead of its own."""
    pages = (SHARED_PREFIX_TOKENS - SINK) // 16
    users = [b for b in sharers if max(SINK, int(lens[b]) - RECENT) // 16 - SINK // 16 >= pages]
    if not users:
        return 0, 0, 0
    per_block = 16 * ((G + 3) // 4)
    reads = -(-len(users) * G // per_block)
    return pages, len(users), (len(users) - reads) * pages * H


def bench_single(rng, gen, dev):
    """One Qwen3-8B-shaped layer at batch 1 and 100,000 tokens: decode_attn over
    8 separate cache copies in turn (525 MB, twice the 256 MB MALL), so every
    call reads its pages from HBM."""
    import torch

    import int2_rotated_kv_write_amd as lib
    from synth.device import sample_queries_device
    name = "qwen3_8b_layer_100k"
    W = build_workload(name, rng, gen, dev)
    q = sample_queries_device(W.B, W.Hq, gen, dev)
    lens_d = torch.from_numpy(W.lens.astype(np.int32)).to(dev)
    out = torch.empty((W.B, W.Hq, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.decode_workspace_bytes(W.shape, W.B, W.max_pages), dtype=torch.uint8, device=dev)
    calls = [lib.prepare_decode_attn(W.shape, c, q, W.table_d, lens_d, out, ws, SIG) for c in W.caches]
    mean, med = event_us(calls, 20 * len(calls))
    nbytes = decode_bytes(W.lens, W.H, W.Hq)
    gbs = nbytes / (mean * 1e-6) / 1e9
    log(f"{name}: decode_attn {mean:.1f} us (median {med:.1f}), {gbs:.0f} GB/s")
    return {"workload": name, "batch": W.B, "seq_len": int(W.lens[0]), "num_q_heads": W.Hq, "num_kv_heads": W.H,
            "page_table": "contiguous", "cache_copies_cycled": W.NL,
            "kernel": "decode_attn (rotate_q + split + reduce)", "us": mean, "us_median": med,
            "bytes_per_launch": nbytes, "achieved_gbs": gbs, "frac": gbs / PEAK_HBM_GBS,
            "tokens_per_s_36_layers": 1.0 / (36 * mean * 1e-6)}


def bench_ragged(rng, gen, dev):
    """64 sequences of 4,096..131,072 tokens, G = 8, a contiguous quarter of the
    batch sharing a 4,096-token prefix (same physical pages): decode_attn, and
    decode_attn_cascade with that quarter as one group."""
    import torch

    import int2_rotated_kv_write_amd as lib
    from synth.device import sample_queries_device
    name = "ragged_64x4k_128k"
    W = build_workload(name, rng, gen, dev)
    G = W.Hq // W.H
    q = sample_queries_device(W.B, W.Hq, gen, dev)
    lens_d = torch.from_numpy(W.lens.astype(np.int32)).to(dev)
    out = torch.empty((W.B, W.Hq, 128), dtype=torch.bfloat16, device=dev)
    out_c = torch.empty_like(out)
    ws = torch.empty(lib.decode_workspace_bytes(W.shape, W.B, W.max_pages), dtype=torch.uint8, device=dev)
    sh_pages = (SHARED_PREFIX_TOKENS - SINK) // 16
    ws_c = torch.empty(lib.cascade_workspace_bytes(W.shape, W.B, W.max_pages, sh_pages), dtype=torch.uint8,
                       device=dev)
    s0, n_sh = W.sharers[0], len(W.sharers)
    cu = torch.tensor([s0, s0 + n_sh], dtype=torch.int32, device=dev)
    gp = torch.tensor([sh_pages], dtype=torch.int32, device=dev)
    plain = lib.prepare_decode_attn(W.shape, W.caches[0], q, W.table_d, lens_d, out, ws, SIG)
    cas = lib.prepare_decode_attn_cascade(W.shape, W.caches[0], q, W.table_d, lens_d, cu, gp, out_c, ws_c, n_sh,
                                          sh_pages, SIG)
    t_plain, m_plain = event_us([plain], 20)
    t_cas, m_cas = event_us([cas], 20)
    diff = (out.float() - out_c.float()).abs().max().item()
    nbytes = decode_bytes(W.lens, W.H, W.Hq)
    pages, users, saved_blocks = shared_pages_saved(W.lens, W.sharers, W.H, G)
    saved = saved_blocks * 1280
    gbs = nbytes / (t_plain * 1e-6) / 1e9
    log(f"{name}: decode_attn {t_plain:.1f} us ({gbs:.0f} GB/s), cascade {t_cas:.1f} us, "
        f"{saved / 1e6:.1f} MB of shared pages not re-read, max |out diff| {diff:.3g}")
    return {"workload": name, "batch": W.B, "seq_len_min": int(W.lens.min()), "seq_len_max": int(W.lens.max()),
            "seq_len_total": int(W.lens.sum()), "num_q_heads": W.Hq, "num_kv_heads": W.H,
            "page_table": "permuted, shared prefix", "sharers": n_sh, "shared_prefix_tokens": SHARED_PREFIX_TOKENS,
            "decode_attn": {"us": t_plain, "us_median": m_plain, "bytes_per_launch": nbytes, "achieved_gbs": gbs,
                            "frac": gbs / PEAK_HBM_GBS},
            "decode_attn_cascade": {"us": t_cas, "us_median": m_cas, "bytes_per_launch": nbytes - saved,
                                    "shared_int2_pages": pages, "sharers_using_shared_reads": users,
                                    "page_bytes_saved": saved, "bytes_saved_frac": saved / nbytes,
                                    "speedup": t_plain / t_cas, "max_abs_diff_vs_decode_attn": diff}}


ABLATION = dict(batch=8, seq_len=16384, q_heads=8, kv_heads=2, rank=8)


def naive_basis():
    """U = P H (Sylvester Hadamard / sqrt(128), rows in 7-bit-reversed order), so that
    R = U H P = P H H P = I: INT2 then quantizes the raw channels (the naive
    INT2 baseline), up to the bf16 rounding of U."""
    h = np.array([[1.0]])
    while h.shape[0] < 128:
        h = np.block([[h, h], [h, -h]])
    br = [int(format(i, "07b")[::-1], 2) for i in range(128)]
    return h[br, :] / math.sqrt(128)



def bench_extend(rng, gen, dev):
    """Chunked prefill at long context: EXTEND_CHUNK new tokens of one sequence (32 query /
    8 KV heads) attend to its cached 100,000-token prefix as stored (INT2 history through
    the folded rotation, BF16 sink and ring) and causally to their own keys, in one
    extend_attn call.  Its work is counted as the attention's QK and PV products (4 x 128
    flops per query head and key) against the dense fp16 MFMA peak; the bytes are the
    prefix cache read once plus the chunk's q, k, v and out."""
    import torch

    import int2_rotated_kv_write_amd as lib
    from synth.device import sample_kv_device, sample_queries_device
    name = "extend_1x100k_chunk1024"
    W = build_workload(name, rng, gen, dev)
    T, P = EXTEND_CHUNK, int(W.lens[0])
    q = sample_queries_device(T, W.Hq, gen, dev)
    k = sample_kv_device(W.law, T, gen, dev)
    v = sample_kv_device(W.law, T, gen, dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    prefix = torch.tensor([P], dtype=torch.int32, device=dev)
    out = torch.empty((T, W.Hq, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.extend_workspace_bytes(W.shape, T, W.max_pages, T), dtype=torch.uint8, device=dev)
    call = lambda: lib.extend_attn(W.shape, W.caches[0], q, k, v, cu, prefix, W.table_d, out, ws, T, SIG)
    mean, med = event_us([call], 10)
    keys = T * P + T * (T + 1) // 2                  # (query row, key) pairs per query head
    flops = 4 * 128 * W.Hq * keys
    nbytes = decode_bytes(W.lens, W.H, W.Hq) - W.Hq * 128 * 2 * 2 + T * (W.Hq * 2 + W.H * 2) * 128 * 2
    tflops = flops / (mean * 1e-6) / 1e12
    log(f"{name}: extend_attn {mean:.1f} us (median {med:.1f}), {tflops:.1f} TFLOP/s")
    return {"workload": name, "batch": 1, "prefix_len": P, "chunk_len": T, "num_q_heads": W.Hq,
            "num_kv_heads": W.H, "page_table": "permuted",
            "kernel": "extend_attn (rotate_q, extend INT2 ranges, extend BF16 rows, reduce)", "us": mean,
            "us_median": med, "flops": flops, "achieved_tflops": tflops, "peak_tflops": PEAK_F16_MFMA_TFLOPS,
            "frac": tflops / PEAK_F16_MFMA_TFLOPS, "bytes": nbytes,
            "achieved_gbs": nbytes / (mean * 1e-6) / 1e9}


def bench_group128(rng, gen, dev):
    """decode_attn at 28 x 100K in the 2.25-bit format (one fp16 scale and zero per
    token and head), 36 layers' caches cycled as in the headline, and one kv_write
    of 100,000 prefill tokens x 8 KV heads in that format."""
    import torch

    import int2_rotated_kv_write_amd as lib
    import synth
    from synth.device import sample_kv_device, sample_queries_device
    name = "concurrent_28x100k_group128"
    W = build_workload(name, rng, gen, dev)
    q = sample_queries_device(W.B, W.Hq, gen, dev)
    lens_d = torch.from_numpy(W.lens.astype(np.int32)).to(dev)
    out = torch.empty((W.B, W.Hq, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.decode_workspace_bytes(W.shape, W.B, W.max_pages), dtype=torch.uint8, device=dev)
    calls = [lib.prepare_decode_attn(W.shape, c, q, W.table_d, lens_d, out, ws, SIG) for c in W.caches]
    mean, med = event_us(calls, 3 * len(calls))   # as the headline: 3 passes over the layers
    nbytes = decode_bytes(W.lens, W.H, W.Hq, group=128)
    gbs = nbytes / (mean * 1e-6) / 1e9
    u_k, u_v, ck, cv = W.caches[0].u_k, W.caches[0].u_v, W.caches[0].clip_k, W.caches[0].clip_v
    W.caches = None
    torch.cuda.empty_cache()
    n_pre = PREFILL_TOKENS
    pre_pages = math.ceil(n_pre / 16)
    pre_cache = lib.allocate_cache(W.shape, pre_pages, 1, dev, u_k=u_k, u_v=u_v, clip_k=ck, clip_v=cv)
    pre_k = sample_kv_device(W.law, n_pre, gen, dev)
    pre_v = sample_kv_device(W.law, n_pre, gen, dev)
    pre_table = torch.arange(pre_pages, dtype=torch.int32, device=dev).view(1, pre_pages)
    pre_write = lib.prepare_kv_write(W.shape, pre_cache, pre_k, pre_v,
                                     torch.zeros(n_pre, dtype=torch.int32, device=dev),
                                     torch.arange(n_pre, dtype=torch.int32, device=dev), pre_table,
                                     torch.tensor([n_pre], dtype=torch.int32, device=dev))
    w_mean, _ = event_us([pre_write], 10)
    w_bytes = prefill_write_bytes(n_pre, W.H, group=128)
    log(f"{name}: decode_attn {mean:.1f} us ({gbs:.0f} GB/s), kv_write prefill {w_mean:.1f} us")
    return {"workload": name, "batch": W.B, "seq_len": int(W.lens[0]), "num_q_heads": W.Hq, "num_kv_heads": W.H,
            "group": 128, "bits_per_element": 2.25, "layers_cycled": W.NL,
            "decode_attn": {"us": mean, "us_median": med, "bytes_per_launch": nbytes, "achieved_gbs": gbs,
                            "frac": gbs / PEAK_HBM_GBS},
            "kv_write_prefill": {"tokens": n_pre, "us": w_mean, "bytes": w_bytes,
                                 "achieved_gbs": w_bytes / (w_mean * 1e-6) / 1e9}}

def bench_ablation(rng, gen, dev):
    """Attention-output error against BF16 attention of three rotations, all through
    kv_write + decode_attn with only U and the clips changed: OSCAR (calibrated U_Q,
    U_S), Hadamard-only (U = I) and naive INT2 (U = bf16(P H), R ~ I); clips are the
    0.999 quantile of the calibration set rotated by each U.  Three synthetic laws:
    the outlier law with N(0,1) queries; the same K/V with rank-8 queries whose
    directions avoid the outlier channels; and the outlier law turned by a random
    orthogonal matrix per head (outliers along dense directions) with N(0,1)
    queries.  The reference is fp32 softmax attention over the same bf16 K/V."""
    import torch

    import int2_rotated_kv_write_amd as lib
    import synth
    from synth.device import sample_kv_device
    B, L, Hq, H = ABLATION["batch"], ABLATION["seq_len"], ABLATION["q_heads"], ABLATION["kv_heads"]
    G = Hq // H
    shape = lib.CacheShape(H, Hq)
    pages = L // 16
    table_d = torch.arange(B * pages, dtype=torch.int32, device=dev).view(B, pages)
    lens_d = torch.full((B,), L, dtype=torch.int32, device=dev)
    seq = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(L)
    pos = torch.arange(L, dtype=torch.int32, device=dev).repeat(B)
    ws = torch.empty(lib.decode_workspace_bytes(shape, B, pages), dtype=torch.uint8, device=dev)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    eye = synth.f32_to_bf16_bits(np.broadcast_to(np.eye(128), (H, 128, 128)))
    naive = synth.f32_to_bf16_bits(np.broadcast_to(naive_basis(), (H, 128, 128)))
    result = {"setup": {"batch": B, "seq_len": L, "num_q_heads": Hq, "num_kv_heads": H,
                        "calibration_samples": 2048, "clip_quantile": 0.999, "query_rank": ABLATION["rank"],
                        "metric": "||out - ref||_F / ||ref||_F and mean |out - ref| over all outputs; "
                                  "ref = fp32 attention over the bf16 K/V"}}
    for law_name in ("outlier_iid_queries", "outlier_lowrank_misaligned_queries", "dense_outlier_iid_queries"):
        kv_law = synth.dense_outlier_law(rng, H) if law_name.startswith("dense") else synth.outlier_law(rng, H)
        q_law = synth.lowrank_query_law(rng, kv_law, ABLATION["rank"]) if "lowrank" in law_name else None
        qc, kc, vc = synth.calibration_samples(rng, kv_law, G, 2048, q_law)
        u_k, u_v, ck, cv = lib.calibrate_layer(qc, kc, vc, SIG, 0.999)
        variants = {"oscar": (u_k, u_v, ck, cv),
                    "hadamard_only": (eye, eye, lib.calibrate_clip(kc, eye), lib.calibrate_clip(vc, eye)),
                    "naive_int2": (naive, naive, lib.calibrate_clip(kc, naive), lib.calibrate_clip(vc, naive))}
        k = sample_kv_device(kv_law, B * L, gen, dev)
        v = sample_kv_device(kv_law, B * L, gen, dev)
        if q_law is None:
            q = torch.randn((B, Hq, 128), generator=gen, device=dev).to(torch.bfloat16)
        else:
            q = bf(q_law.decode_queries(rng, B, Hq))
        ref = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        kf, vf = k.float().view(B, L, H, 128), v.float().view(B, L, H, 128)
        for b in range(B):
            for h in range(H):
                lg = (q[b, h * G:(h + 1) * G].float() @ kf[b, :, h].t().contiguous()) * SIG
                ref[b, h * G:(h + 1) * G] = torch.softmax(lg, dim=-1) @ vf[b, :, h]
        res = {}
        for name, (uk, uv, c_k, c_v) in variants.items():
            cache = lib.allocate_cache(shape, B * pages, B, dev, u_k=bf(uk), u_v=bf(uv), clip_k=float(c_k),
                                       clip_v=float(c_v))
            lib.kv_write(shape, cache, k, v, seq, pos, table_d, lens_d)
            out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
            lib.decode_attn(shape, cache, q, table_d, lens_d, out, ws, SIG)
            err = out.float() - ref
            res[name] = {"rel_fro_err": (err.norm() / ref.norm()).item(), "mean_abs_err": err.abs().mean().item(),
                         "max_abs_err": err.abs().max().item(), "clip_k": float(c_k), "clip_v": float(c_v)}
            del cache
        for name in res:
            res[name]["err_vs_oscar"] = res[name]["rel_fro_err"] / res["oscar"]["rel_fro_err"]
        log(f"ablation {law_name}: " + ", ".join(f"{n} {r['rel_fro_err']:.4f}" for n, r in res.items()))
        result[law_name] = res
    return result

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="concurrent_28x100k_36l", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the single-sequence and ragged workloads and the rotation ablation")
    ap.add_argument("--only-ablation", action="store_true", help="run the rotation ablation alone and print it")
    ap.add_argument("--only-extend", action="store_true", help="run the chunked-prefill measurement alone and print it")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this build is single-GPU: the decode shards by sequence or KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import int2_rotated_kv_write_amd as lib
    import synth
    from synth.device import sample_kv_device, sample_queries_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    lib.load()
    if args.only_ablation or args.only_extend:
        rng = np.random.default_rng(args.seed)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        if args.only_ablation:
            print(json.dumps({"rotation_ablation": bench_ablation(rng, gen, dev)}), flush=True)
        else:
            print(json.dumps({"extend_1x100k_chunk1024": bench_extend(rng, gen, dev)}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    rng = np.random.default_rng(args.seed)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    W = build_workload(args.workload, rng, gen, dev, n_fill_minus=1)
    B, Hq, H, NL = W.B, W.Hq, W.H, W.NL
    lens, max_pages, shape, law, table_d, caches = W.lens, W.max_pages, W.shape, W.law, W.table_d, W.caches
    num_pages = W.num_pages
    # ---- per-step inputs: the new token of every sequence and the queries ----
    new_k = [sample_kv_device(law, B, gen, dev) for _ in range(NL)]
    new_v = [sample_kv_device(law, B, gen, dev) for _ in range(NL)]
    qs = [sample_queries_device(B, Hq, gen, dev) for _ in range(NL)]
    seq_idx = torch.arange(B, dtype=torch.int32, device=dev)
    new_pos = torch.from_numpy((lens - 1).astype(np.int32)).to(dev)
    lens_d = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.decode_workspace_bytes(shape, B, max_pages), dtype=torch.uint8, device=dev)
    # reference kernel of known size for calibrating HBM counters (a kernel
    # nothing else launches): reads and writes 256 MiB once, untimed
    ref_src = torch.ones(32 << 20, dtype=torch.int64, device=dev)
    ref_dst = torch.empty_like(ref_src)
    torch.bitwise_not(ref_src, out=ref_dst)
    del ref_src, ref_dst
    # one layer of the step: decode_step = kv_write of every sequence's new token, then
    # decode_attn over all 100,000 tokens (one call; the writes share a launch with the
    # query rotation)
    layer_steps = [lib.prepare_decode_step(shape, caches[l], new_k[l], new_v[l], seq_idx, new_pos, lens_d, qs[l],
                                           table_d, lens_d, out, ws, SIG) for l in range(NL)]
    decodes = [lib.prepare_decode_attn(shape, caches[l], qs[l], table_d, lens_d, out, ws, SIG)
               for l in range(NL)]
    torch.cuda.synchronize()

    def step():
        for l in range(NL):
            layer_steps[l]()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # decode_attn alone (the roofline kernel): HIP events on the stream the library
    # launches on (torch's current stream) around each call, 3 passes over the layers
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3 * NL)]
    for l in range(NL):
        decodes[l]()
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        decodes[i % NL]()
        e1.record()
    torch.cuda.synchronize()
    dec_ms = [e0.elapsed_time(e1) for e0, e1 in ev]

    ms_per_step = 1e3 * elapsed / args.steps
    tok_s = B * args.steps / elapsed
    group = wl.get("group", 64)
    dbytes = decode_bytes(lens, H, Hq, group)
    wbytes = write_bytes(B, H, group)
    step_bytes = NL * (dbytes + wbytes)
    dec_avg_ms = statistics.mean(dec_ms)
    achieved = dbytes / (dec_avg_ms * 1e-3) / 1e9
    log(f"step {ms_per_step:.3f} ms, decode_attn avg {dec_avg_ms * 1e3:.1f} us/layer, "
        f"{achieved:.0f} GB/s decode, {step_bytes / (elapsed / args.steps) / 1e9:.0f} GB/s step")

    # ---- write path: one kv_write of 100,000 prefill tokens x H KV heads (K and V),
    # outlier law, its own calibration; HIP events around each call ----
    W.caches = None
    del caches, layer_steps, decodes
    torch.cuda.empty_cache()
    pw_law = synth.outlier_law(rng, H)
    pqc, pkc, pvc = synth.calibration_samples(rng, pw_law, Hq // H, 2048)
    pu_k, pu_v, pck, pcv = lib.calibrate_layer(pqc, pkc, pvc, SIG, 0.999)
    n_pre = PREFILL_TOKENS
    pre_pages = math.ceil(n_pre / 16)
    pre_cache = lib.allocate_cache(shape, pre_pages, 1, dev, u_k=bf(pu_k), u_v=bf(pu_v),
                                   clip_k=float(pck), clip_v=float(pcv))
    pre_k = sample_kv_device(pw_law, n_pre, gen, dev)
    pre_v = sample_kv_device(pw_law, n_pre, gen, dev)
    pre_table = torch.arange(pre_pages, dtype=torch.int32, device=dev).view(1, pre_pages)
    pre_write = lib.prepare_kv_write(shape, pre_cache, pre_k, pre_v,
                                     torch.zeros(n_pre, dtype=torch.int32, device=dev),
                                     torch.arange(n_pre, dtype=torch.int32, device=dev), pre_table,
                                     torch.tensor([n_pre], dtype=torch.int32, device=dev))
    for _ in range(2):
        pre_write()
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e0, e1 in pev:
        e0.record()
        pre_write()
        e1.record()
    torch.cuda.synchronize()
    pre_us = 1e3 * statistics.mean(e0.elapsed_time(e1) for e0, e1 in pev)
    pre_bytes = prefill_write_bytes(n_pre, H, group=group)
    pre_gbs = pre_bytes / (pre_us * 1e-6) / 1e9
    log(f"kv_write prefill of {n_pre} tokens x {H} heads: {pre_us:.1f} us, {pre_gbs:.0f} GB/s")
    del pre_cache, pre_k, pre_v

    # ---- the BF16 baseline: the same sequences, heads and page table in an
    # all-BF16 paged cache, one bf16_decode_attn per layer; HIP events ----
    from synth.device import fill_bf16_pages_device
    torch.cuda.empty_cache()
    b16_pages = torch.zeros((num_pages, H, 4096), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        L = int(lens[b])
        if L:
            fill_bf16_pages_device(b16_pages, sample_kv_device(law, L, gen, dev), sample_kv_device(law, L, gen, dev),
                                   table_d[b])
    b16_ws = torch.empty(lib.bf16_decode_workspace_bytes(H, Hq, B, max_pages), dtype=torch.uint8, device=dev)
    b16_call = lib.prepare_bf16_decode_attn(H, Hq, b16_pages, qs[0], table_d, lens_d, out, b16_ws, SIG)
    for _ in range(2):
        b16_call()
    bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e0, e1 in bev:
        e0.record()
        b16_call()
        e1.record()
    torch.cuda.synchronize()
    b16_us = 1e3 * statistics.mean(e0.elapsed_time(e1) for e0, e1 in bev)
    b16_bytes = bf16_decode_bytes(lens, H, Hq)
    b16_gbs = b16_bytes / (b16_us * 1e-6) / 1e9
    log(f"bf16 baseline decode: {b16_us:.1f} us/layer, {b16_gbs:.0f} GB/s; "
        f"INT2 decode_attn is {b16_us / (dec_avg_ms * 1e3):.2f}x faster")
    del b16_pages, b16_ws, b16_call

    # ---- practical read ceiling: one plain stream over 8 GiB (library probe) ----
    torch.cuda.empty_cache()
    probe_buf = torch.ones(8 << 30, dtype=torch.uint8, device=dev)
    probe_sink = torch.empty(lib.read_probe_sink_bytes(), dtype=torch.uint8, device=dev)
    probe = lib.prepare_read_probe(probe_buf, probe_sink)
    probe()
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for e0, e1 in rev:
        e0.record()
        probe()
        e1.record()
    torch.cuda.synchronize()
    read_gbs = (8 << 30) / (1e-3 * statistics.median(e0.elapsed_time(e1) for e0, e1 in rev)) / 1e9
    log(f"read probe: {read_gbs:.0f} GB/s (decode_attn at {achieved / read_gbs:.1%} of it)")
    del probe_buf, probe_sink, probe

    extras = {}
    if not args.no_extras:
        torch.cuda.empty_cache()
        extras["single_1x100k"] = bench_single(rng, gen, dev)
        torch.cuda.empty_cache()
        extras["ragged_64x4k_128k"] = bench_ragged(rng, gen, dev)
        torch.cuda.empty_cache()
        extras["concurrent_28x100k_group128"] = bench_group128(rng, gen, dev)
        torch.cuda.empty_cache()
        extras["extend_1x100k_chunk1024"] = bench_extend(rng, gen, dev)
        torch.cuda.empty_cache()
        extras["rotation_ablation"] = bench_ablation(rng, gen, dev)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        t_unit, reps, threads, t_one, reps_one = cpu_baseline(H, NL, int(lens.max()))
        units = B * H * NL
        cpu = {"value": B / (t_unit * units), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
               "sample": (f"fp64 oracle decode of 1 sequence x 1 KV head (4 query heads) at "
                          f"L={int(lens.max())}, median of {reps} runs = {t_unit:.3f}s with {threads} BLAS "
                          f"threads, extrapolated x{units} (batch x KV heads x layers)"),
               "one_thread": {"value": B / (t_one * units), "unit": "tokens/s", "cores": 1,
                              "sample": f"the same unit with 1 BLAS thread, median of {reps_one} runs = {t_one:.3f}s"}}
        log(f"cpu baseline: {t_unit:.3f}s per unit with {threads} threads, {t_one:.3f}s with 1")

    traffic = None
    if args.workload == "concurrent_28x100k_36l":
        traffic = read_traffic()

    rec = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int2 codes x f16 -> f32", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "seq_len": int(lens.max()) if B else 0,
                   "seq_len_total": int(lens.sum()), "num_q_heads": Hq, "num_kv_heads": H,
                   "head_dim": 128, "layers": NL, "page_size": 16, "page_table": wl["table"],
                   "sink": 64, "recent": 256,
                   "step": "per layer: decode_step = kv_write(1 token/seq) then decode_attn, one call"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "decode_attn (rotate_q + split + reduce), per layer",
                     "bytes_per_launch": dbytes, "avg_launch_us": dec_avg_ms * 1e3,
                     "practical_read_gbs": read_gbs, "frac_of_practical": achieved / read_gbs},
        "kv_write_prefill": {"tokens": n_pre, "kv_heads": H, "us": pre_us, "tokens_per_s": n_pre / (pre_us * 1e-6),
                             "bytes": pre_bytes, "achieved_gbs": pre_gbs, "frac": pre_gbs / PEAK_HBM_GBS},
        "bf16_baseline": {"kernel": "bf16_decode_attn (split + reduce) over an all-BF16 paged cache, per layer",
                          "us": b16_us, "bytes": b16_bytes, "achieved_gbs": b16_gbs,
                          "frac": b16_gbs / PEAK_HBM_GBS, "int2_speedup": b16_us / (dec_avg_ms * 1e3),
                          "cache_bytes_ratio": b16_bytes / dbytes},
        "step_hbm_gbs": step_bytes / (elapsed / args.steps) / 1e9,
        **extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
