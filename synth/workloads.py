"""Seeded synthetic workloads: token K/V, queries, calibration samples, page tables.

Distributions follow the workload descriptions the library is measured on:

* "outlier" law: every channel N(0,1), except a few fixed channels per KV head
  that are scaled x20 (the channel-outlier problem both the Italian and the
  Spanish page describe as the reason INT2 fails without rotation).
* "heavy" law: N(0,1) with 2% of the 128 channels per head (ceil -> 3 channels)
  drawn from a Student-t with nu=3, scaled x10.

Everything is drawn from ``numpy.random.Generator(PCG64(seed))`` so the oracle
and the GPU path see bit-identical bf16 inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128

__all__ = [
    "HEAD_DIM", "f32_to_bf16_bits", "bf16_bits_to_f32", "KVLaw", "outlier_law",
    "heavy_tail_law", "calibration_samples", "decode_queries", "QueryLaw", "lowrank_query_law",
    "dense_outlier_law",
    "contiguous_page_table", "permuted_page_table", "shared_prefix_page_table",
    "ragged_lengths", "WORKLOADS",
]


# ----------------------------------------------------------------------------
# bf16 storage of samples (input preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# K/V sample laws
# ----------------------------------------------------------------------------
@dataclass
class KVLaw:
    """A per-KV-head channel law: which channels are special and how."""
    kind: str                      # "outlier" or "heavy"
    channels: np.ndarray           # [H_kv][n_special] channel indices
    scale: float = 20.0
    nu: float = 3.0
    mix: np.ndarray | None = None  # [H_kv][128][128] orthogonal: samples x -> x mix (dense outlier directions)

    @property
    def num_heads(self) -> int:
        return int(self.channels.shape[0])

    def sample(self, rng: np.random.Generator, n_tokens: int) -> np.ndarray:
        """float32 [n_tokens][H_kv][128]."""
        H = self.num_heads
        x = rng.standard_normal((n_tokens, H, HEAD_DIM), dtype=np.float32)
        for h in range(H):
            ch = self.channels[h]
            if self.kind == "outlier":
                x[:, h, ch] *= np.float32(self.scale)
            elif self.kind == "heavy":
                t = rng.standard_t(self.nu, size=(n_tokens, len(ch)))
                x[:, h, ch] = (t * self.scale).astype(np.float32)
            else:
                raise ValueError(self.kind)
        if self.mix is not None:
            x = np.einsum("nhc,hcd->nhd", x, self.mix).astype(np.float32)
        return x

    def sample_bf16(self, rng: np.random.Generator, n_tokens: int) -> np.ndarray:
        """uint16 bf16 bits [n_tokens][H_kv][128]."""
        return f32_to_bf16_bits(self.sample(rng, n_tokens))


def outlier_law(rng: np.random.Generator, num_heads: int, n_channels: int = 4,
                scale: float = 20.0) -> KVLaw:
    ch = np.stack([np.sort(rng.choice(HEAD_DIM, n_channels, replace=False))
                   for _ in range(num_heads)])
    return KVLaw("outlier", ch, scale=scale)


def dense_outlier_law(rng: np.random.Generator, num_heads: int, n_channels: int = 4,
                      scale: float = 20.0) -> KVLaw:
    """The outlier law seen through a random orthogonal matrix per head: the
    x20 outliers lie along dense directions instead of single channels."""
    base = outlier_law(rng, num_heads, n_channels, scale)
    mix = np.stack([np.linalg.qr(rng.standard_normal((HEAD_DIM, HEAD_DIM)))[0] for _ in range(num_heads)])
    return KVLaw("outlier", base.channels, scale=scale, mix=mix)


def heavy_tail_law(rng: np.random.Generator, num_heads: int, frac: float = 0.02,
                   scale: float = 10.0, nu: float = 3.0) -> KVLaw:
    n = int(math.ceil(frac * HEAD_DIM))  # 2.56 -> 3 channels per head
    ch = np.stack([np.sort(rng.choice(HEAD_DIM, n, replace=False))
                   for _ in range(num_heads)])
    return KVLaw("heavy", ch, scale=scale, nu=nu)


@dataclass
class QueryLaw:
    """Anisotropic queries: per KV head, q = z B + noise e with z ~ N(0, (128/r) I_r)
    over an orthonormal basis B of r directions (rows) and e ~ N(0, I), so that
    E|q|^2 is about 128 as for N(0,1) queries but concentrated in r directions."""
    basis: np.ndarray              # [H_kv][r][128]
    noise: float = 0.05

    def sample(self, rng: np.random.Generator, num_heads_per_kv: int, n: int) -> np.ndarray:
        """float32 [H_kv][G][n][128]."""
        H, r, _ = self.basis.shape
        z = rng.standard_normal((H, num_heads_per_kv, n, r)) * math.sqrt(HEAD_DIM / r)
        q = np.einsum("hgnr,hrd->hgnd", z, self.basis)
        q += self.noise * rng.standard_normal(q.shape)
        return q.astype(np.float32)

    def decode_queries(self, rng: np.random.Generator, batch: int, num_q_heads: int) -> np.ndarray:
        """bf16 bits [B][Hq][128]; query head h G + g follows KV head h's basis."""
        H = self.basis.shape[0]
        G = num_q_heads // H
        q = self.sample(rng, G, batch)                       # [H][G][B][128]
        return f32_to_bf16_bits(q.transpose(2, 0, 1, 3).reshape(batch, num_q_heads, HEAD_DIM))


def lowrank_query_law(rng: np.random.Generator, kv_law: KVLaw, rank: int = 8, noise: float = 0.05) -> QueryLaw:
    """Queries of rank `rank` per KV head whose directions avoid the K/V law's
    special channels (random Gaussian directions with those channels zeroed,
    then orthonormalised): low-rank and misaligned with the outliers."""
    bases = []
    for h in range(kv_law.num_heads):
        a = rng.standard_normal((HEAD_DIM, rank))
        a[kv_law.channels[h], :] = 0.0
        qmat, _ = np.linalg.qr(a)
        bases.append(qmat.T)
    return QueryLaw(np.stack(bases), noise)


def calibration_samples(rng: np.random.Generator, law: KVLaw, group_size: int,
                        n_samples: int = 2048, q_law: QueryLaw | None = None):
    """Calibration activations for one layer.

    Returns float64 arrays (q_cal [H][G][N][128] ~ N(0,1), or from ``q_law``,
    k_cal [H][N][128], v_cal [H][N][128]) with K and V drawn from ``law``, each
    value rounded to bf16 first (they stand in for activations a bf16 model
    would produce).
    """
    H = law.num_heads
    if q_law is None:
        q = rng.standard_normal((H, group_size, n_samples, HEAD_DIM), dtype=np.float32)
    else:
        q = q_law.sample(rng, group_size, n_samples)
    q = bf16_bits_to_f32(f32_to_bf16_bits(q)).astype(np.float64)
    k = law.sample(rng, n_samples).transpose(1, 0, 2)
    v = law.sample(rng, n_samples).transpose(1, 0, 2)
    k = bf16_bits_to_f32(f32_to_bf16_bits(k)).astype(np.float64)
    v = bf16_bits_to_f32(f32_to_bf16_bits(v)).astype(np.float64)
    return q, np.ascontiguousarray(k), np.ascontiguousarray(v)


def decode_queries(rng: np.random.Generator, batch: int, num_q_heads: int) -> np.ndarray:
    """bf16 bits [B][Hq][128], N(0,1)."""
    q = rng.standard_normal((batch, num_q_heads, HEAD_DIM), dtype=np.float32)
    return f32_to_bf16_bits(q)


# ----------------------------------------------------------------------------
# page tables and lengths
# ----------------------------------------------------------------------------
def contiguous_page_table(batch: int, max_pages: int) -> np.ndarray:
    """Sequence b owns physical pages [b*max_pages, (b+1)*max_pages) in order."""
    return (np.arange(batch * max_pages, dtype=np.int32)).reshape(batch, max_pages)


def permuted_page_table(rng: np.random.Generator, batch: int, max_pages: int,
                        num_pages: int | None = None) -> np.ndarray:
    """Each sequence's logical pages map to a random, disjoint set of physical pages."""
    total = batch * max_pages
    num_pages = total if num_pages is None else num_pages
    if num_pages < total:
        raise ValueError("pool too small")
    perm = rng.permutation(num_pages)[:total].astype(np.int32)
    return perm.reshape(batch, max_pages)


def shared_prefix_page_table(rng: np.random.Generator, lens, max_pages: int,
                             prefix_tokens: int, sharers, page_size: int = 16):
    """Permuted table where the sequences in ``sharers`` share the physical pages of
    the first ``prefix_tokens`` tokens (a prefix-cache hit).  The first sharer
    owns those pages; the others point at them.  Returns (table, num_pages,
    owner) where owner[b] is the sequence whose pages hold b's prefix.
    """
    B = len(lens)
    need = [int(math.ceil(L / page_size)) for L in lens]
    pp = prefix_tokens // page_size
    sharers = list(sharers)
    total = sum(need) - pp * max(0, len(sharers) - 1)
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    owner = np.arange(B)
    cur = 0
    shared_pages = None
    for b in range(B):
        n = need[b]
        if b in sharers and shared_pages is not None:
            table[b, :pp] = shared_pages
            table[b, pp:n] = perm[cur:cur + n - pp]
            cur += n - pp
            owner[b] = sharers[0]
        else:
            table[b, :n] = perm[cur:cur + n]
            cur += n
            if b in sharers:
                shared_pages = table[b, :pp].copy()
    assert cur == total
    # unused tail entries point at page 0 (never read: beyond the length)
    table[table < 0] = 0
    return table, total, owner


def ragged_lengths(rng: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


# ----------------------------------------------------------------------------
# Named workloads (shapes of the configurations the library is measured on)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_kv_heads: int
    num_q_heads: int
    seq_len: int | tuple = 0
    layers: int = 1
    law: str = "outlier"
    table: str = "contiguous"
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # 1 sequence, 1 KV head, 4 query heads, 1024 tokens (64 sink / 704 INT2 / 256 recent)
    "tiny_gqa4_1k": Workload("tiny_gqa4_1k", 1, 1, 4, 1024, law="outlier"),
    # one Qwen3-8B-shaped layer: 32 q / 8 kv heads, 100,000 tokens, contiguous pages
    "qwen3_8b_layer_100k": Workload("qwen3_8b_layer_100k", 1, 8, 32, 100_000, law="heavy"),
    # write path: 100,000 prefill tokens x 8 KV heads, K and V
    "prefill_write_100k": Workload("prefill_write_100k", 1, 8, 32, 100_000, law="outlier"),
    # 28 concurrent 100,000-token sequences, 36 layers, permuted pages
    "concurrent_28x100k_36l": Workload("concurrent_28x100k_36l", 28, 8, 32, 100_000,
                                       layers=36, law="heavy", table="permuted"),
    # 64 ragged sequences in [4096, 131072], 64 q / 8 kv heads, 25% shared prefix
    "ragged_64x4k_128k": Workload("ragged_64x4k_128k", 64, 8, 64, (4096, 131072),
                                  law="outlier", table="shared_prefix",
                                  extra={"prefix_tokens": 4096, "n_share": 16}),
}
