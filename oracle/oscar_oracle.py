"""fp64 oracle: OSCAR rotation, INT2 KV write and mixed-precision paged decode.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Plain NumPy, float64
throughout, dense matrices, no blocking or fusion beyond what the definitions
state.

Pages cited (title, then the short tag used below):
  [it] "OSCAR: Come Together AI Comprime la KV Cache a 2-bit per LLM" (ainsights.it)
  [ru] "Together AI vypustila ishodniki OSCAR -- INT2-kvantovanie KV-kesha dlya
       dolgih kontekstov LLM" (edge.aivizor.me; Russian; no section headings,
       cited by paragraph)
  [es] "Resumen Tecnico: OSCAR - Rotacion Consciente de la Covarianza Espectral
       Offline para Cuantizacion de Cache KV de 2 bits" (gist.science 2605.17757)

Readings taken where the pages are silent are listed with each function and
collected in the repository's design notes.

Page block format (one block per physical page id and KV head); the pages
only say the cache is paged, so the layout is this library's own.  With
groups of 64 channels (2 groups per token) the block is 1280 bytes:
  [   0,  512)  K codes, token-major: slot t at byte 32*t; channel j (post-P
                index) at byte j//4, bits 2*(j%4).
  [ 512, 1024)  V codes, channel-major: channel j is the little-endian uint32 at
                512 + 4*j; slot t at bits 2*t.
  [1024, 1152)  K group parameters: slot t at 1024 + 8*t: fp16 s0, z0, s1, z1.
  [1152, 1280)  V group parameters: slot t at 1152 + 8*t: fp16 s0, z0, s1, z1.
With one group of 128 channels per token (2.25 bits per element: the format
behind [ru] paragraph 4's "2.28 bits per KV element") it is 1152 bytes: the
same codes, then K parameters at 1024 + 4*t (fp16 s, z) and V parameters at
1088 + 4*t.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "D", "PAGE_BLOCK", "K_CODES", "V_CODES", "K_PARAMS", "V_PARAMS", "block_layout",
    "Shape", "Cache", "Layer", "bf16_to_f64", "f64_to_bf16", "fp16_rne",
    "hadamard", "bitrev7", "bitrev_permutation", "rotate", "rotation", "quantize",
    "pack_k_codes", "unpack_k_codes", "regions", "kv_write", "gather_sequence",
    "decode", "decode_folded", "extend", "query_covariance", "score_weighted_covariance",
    "eigenbasis", "calibrate_layer", "new_cache", "BF16_BLOCK", "new_bf16_pages",
    "bf16_pages_write", "bf16_pages_gather", "decode_bf16_paged",
]

D = 128                      # head_dim
PAGE_BLOCK = 1280            # block bytes with 64-channel groups
K_CODES, V_CODES, K_PARAMS, V_PARAMS = 0, 512, 1024, 1152


def block_layout(group: int):
    """(block bytes, K params offset, V params offset, parameter bytes per slot)
    of the page block for `group`-channel quantization groups (64 or 128);
    the codes are at K_CODES and V_CODES for both."""
    if group == 64:
        return PAGE_BLOCK, K_PARAMS, V_PARAMS, 8
    if group == 128:
        return 1152, 1024, 1088, 4
    raise ValueError("group must be 64 or 128")


# ----------------------------------------------------------------------------
# configuration
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Shape:
    """Cache geometry.  Sink 64 / recent 256 are the sizes [it] gives in
    "Architettura del Sistema di Serving e Layout di Memoria"; groups of 64
    channels with an fp16 scale and zero per token-group are this build's
    quantizer format (the pages only say "INT2"); group = 128 (one scale and
    zero per token) is the 2.25-bit variant."""
    num_kv_heads: int
    num_q_heads: int
    head_dim: int = 128
    page_size: int = 16
    sink: int = 64
    recent: int = 256
    group: int = 64

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class Cache:
    pages: np.ndarray      # uint8 [num_pages][H_kv][block bytes: 1280, or 1152 with 128-channel groups]
    k_sink: np.ndarray     # uint16 bf16 [slots][H_kv][sink][128]
    v_sink: np.ndarray
    k_ring: np.ndarray     # uint16 bf16 [slots][H_kv][recent][128], row = pos % recent
    v_ring: np.ndarray


@dataclass
class Layer:
    u_k: np.ndarray        # uint16 bf16 bits [H_kv][128][128], rows = input channel
    u_v: np.ndarray
    clip_k: np.float32
    clip_v: np.float32


def new_cache(shape: Shape, num_pages: int, num_slots: int) -> Cache:
    H = shape.num_kv_heads
    return Cache(
        pages=np.zeros((num_pages, H, block_layout(shape.group)[0]), np.uint8),
        k_sink=np.zeros((num_slots, H, shape.sink, D), np.uint16),
        v_sink=np.zeros((num_slots, H, shape.sink, D), np.uint16),
        k_ring=np.zeros((num_slots, H, shape.recent, D), np.uint16),
        v_ring=np.zeros((num_slots, H, shape.recent, D), np.uint16),
    )


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(np.asarray(bits, np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest, ties to even (finite inputs).

    Rounds the float64 directly at the 8-bit significand: x = m * 2**e with
    |m| in [1, 2); the bf16 value keeps 7 fraction bits."""
    x = np.asarray(x, np.float64)
    out = np.zeros(x.shape, np.float64)
    nz = x != 0
    m, e = np.frexp(x[nz])               # x = m * 2**e, 0.5 <= |m| < 1
    # 8 significant bits: scale so the kept bits are the integer part
    scaled = m * 256.0
    r = np.rint(scaled)                   # ties to even
    out[nz] = np.ldexp(r / 256.0, e)
    bits32 = out.astype(np.float32).view(np.uint32)   # exact: 8 significant bits
    return (bits32 >> 16).astype(np.uint16)


def fp16_rne(x) -> np.ndarray:
    """float64 -> IEEE binary16, round to nearest even, as float16.

    NumPy converts float64 to float16 directly (one rounding, not via
    float32); tests/test_oracle_formats.py pins that behaviour."""
    return np.asarray(x, np.float64).astype(np.float16)


# ----------------------------------------------------------------------------
# the three rotation factors ([it] "I tre fattori della rotazione";
# [ru] paragraph 3; [es] section 2.2 A.3 "Construccion de Rotacion Compuesta")
# ----------------------------------------------------------------------------
def hadamard(d: int = D) -> np.ndarray:
    """Orthonormal Walsh-Hadamard matrix H_Had in Sylvester (natural) order.

    Sylvester recursion S_1 = [1], S_2n = [[S_n, S_n], [S_n, -S_n]], then
    H = S_d / sqrt(d).  The normalisation is the one under which the lemma of
    [ru] paragraph 5 (every diagonal entry of H Lambda H^T equals tr(Lambda)/d)
    holds, and makes H orthogonal as [ru] paragraph 2 requires of the rotations.
    """
    S = np.ones((1, 1))
    while S.shape[0] < d:
        S = np.block([[S, S], [S, -S]])
    if S.shape[0] != d:
        raise ValueError("d must be a power of two")
    return S / np.sqrt(d)


def bitrev7(i) -> np.ndarray:
    """Reverse the 7 low bits of i (index of a 128-channel vector)."""
    i = np.asarray(i, np.int64)
    r = np.zeros_like(i)
    for b in range(7):
        r |= ((i >> b) & 1) << (6 - b)
    return r


def bitrev_permutation(d: int = D) -> np.ndarray:
    """P_br with P[i, br(i)] = 1, so (z P)_j = z_{br(j)}.

    [es] 2.2 A.3 names it a bit-reversal permutation that interleaves high- and
    low-variance channels across quantization groups; [it] calls it "Permuted
    Bit-Reversal".  Read as the plain 7-bit index reversal (an involution)."""
    if d != D:
        raise ValueError("bit reversal is defined here for d = 128")
    P = np.zeros((d, d))
    P[np.arange(d), bitrev7(np.arange(d))] = 1.0
    return P


def rotate(x: np.ndarray, u_bits: np.ndarray) -> np.ndarray:
    """x R for row vectors x [..., 128], applying the factors in order:
    y = x U, z = y H with H = S/sqrt(128) (integer Sylvester S first, one
    division after, so exact zeros stay exact), w = z P_br, i.e. w_j =
    z_{br(j)}."""
    U = bf16_to_f64(u_bits)
    S = hadamard(D) * np.sqrt(D)              # exact +-1 entries
    z = ((x @ U) @ np.rint(S)) / np.sqrt(D)
    return z[..., bitrev7(np.arange(D))]


def rotation(u_bits: np.ndarray) -> np.ndarray:
    """R = U . H_Had . P_br for one head, in fp64, from the bf16 U the library
    also receives.  Row-vector convention: a token k is stored as k' = k R
    (covariances are built as q^T q from row vectors, [ru] paragraph 2 and
    [es] 2.2 A.1)."""
    U = bf16_to_f64(u_bits)
    return U @ hadamard(D) @ bitrev_permutation(D)


# ----------------------------------------------------------------------------
# INT2 quantizer (groups of 64 or 128 channels, fp16 scale and fp16 zero per token-group)
# ----------------------------------------------------------------------------
def quantize(w: np.ndarray, group: int = 64):
    """Asymmetric min/max INT2 of already-clipped rotated values.

    For every `group`-channel group (64: two per token, 128: one):
    s = fp16((max - min) / 3), z = fp16(min), and
    code = clamp(rne((w - z) / s), 0, 3), using the fp16-rounded s and z so
    the stored parameters decode what was encoded.  s == 0 gives all-zero
    codes (the group decodes to z).

    Returns (codes uint8 [..,128], s16, z16 float16 [..,G], s_pre, z_pre
    float64 [..,G] before fp16 rounding, t float64 [..,128] before rounding).
    """
    lead = w.shape[:-1]
    ng = w.shape[-1] // group
    seg = w.reshape(lead + (ng, group))
    mn = seg.min(axis=-1)
    mx = seg.max(axis=-1)
    s_pre = (mx - mn) / 3.0
    s16 = fp16_rne(s_pre)
    z16 = fp16_rne(mn)
    s = s16.astype(np.float64)[..., None]
    z = z16.astype(np.float64)[..., None]
    zero = s == 0
    t = (seg - z) / np.where(zero, 1.0, s)
    code = np.clip(np.rint(t), 0, 3)
    code = np.where(zero, 0.0, code).astype(np.uint8)
    return (code.reshape(w.shape), s16, z16, s_pre, mn, t.reshape(w.shape))


def pack_k_codes(codes: np.ndarray) -> np.ndarray:
    """[..,128] codes -> [..,32] bytes; channel j at byte j//4, bits 2*(j%4)."""
    c = codes.reshape(codes.shape[:-1] + (32, 4)).astype(np.uint8)
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def unpack_k_codes(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, np.uint8)[..., None]
    sh = np.array([0, 2, 4, 6], np.uint8)
    return ((b >> sh) & 3).reshape(b.shape[:-2] + (128,))


def regions(L: int, sink: int, recent: int):
    """Token regions of a sequence of length L ([it] "Architettura del Sistema
    di Serving e Layout di Memoria": the first 64 tokens and the last 256
    before the current position stay BF16, the rest is INT2; [es] 2.2 B).

    Returns (sink_range, int2_range, recent_range) as half-open (lo, hi).
    The recent window [max(sink, L - recent), L) includes the newest token."""
    if L <= sink:
        return (0, L), (L, L), (L, L)
    r_lo = max(sink, L - recent)
    return (0, sink), (sink, r_lo), (r_lo, L)


# ----------------------------------------------------------------------------
# write path ([it] layout section: each token is rotated, clipped and quantized)
# ----------------------------------------------------------------------------
def kv_write(shape: Shape, cache: Cache, layer: Layer, k_bits, v_bits, seq_idx,
             pos, page_table, seq_lens_after):
    """Write T tokens into the cache, exactly as the library's kv_write.

    k_bits, v_bits: uint16 bf16 [T][H_kv][128] (either may be None).
    Every token with pos >= sink is quantized into its INT2 slot (also while it
    is still inside the recent window, so nothing is re-encoded when it leaves
    it); pos < sink copies the bf16 row to the sink buffer; pos >=
    max(sink, L_after - recent) copies it to ring row pos % recent.

    Returns a dict of per-token diagnostics {'K': {...}, 'V': {...}} with the
    quantizer's intermediate values (for the near-tie exclusions of tests).
    """
    seq_idx = np.asarray(seq_idx, np.int64)
    pos = np.asarray(pos, np.int64)
    T = len(pos)
    H = shape.num_kv_heads
    S0, W, PG = shape.sink, shape.recent, shape.page_size
    L_after = np.asarray(seq_lens_after, np.int64)[seq_idx] if T else np.zeros(0, np.int64)
    info = {}
    _, k_par, v_par, pb = block_layout(shape.group)
    for name, bits, R_bits, clip, sink_buf, ring_buf, codes_off, par_off in (
            ("K", k_bits, layer.u_k, layer.clip_k, cache.k_sink, cache.k_ring, K_CODES, k_par),
            ("V", v_bits, layer.u_v, layer.clip_v, cache.v_sink, cache.v_ring, V_CODES, v_par)):
        if bits is None or T == 0:
            continue
        bits = np.asarray(bits, np.uint16)
        # bf16 copies
        m_sink = pos < S0
        if m_sink.any():
            sink_buf[seq_idx[m_sink], :, pos[m_sink]] = bits[m_sink]
        m_ring = pos >= np.maximum(S0, L_after - W)
        if m_ring.any():
            ring_buf[seq_idx[m_ring], :, pos[m_ring] % W] = bits[m_ring]
        # INT2
        m_q = pos >= S0
        x = bf16_to_f64(bits[m_q])                        # [Tq][H][128]
        w_raw = np.stack([rotate(x[:, h], R_bits[h]) for h in range(H)], axis=1)
        c = float(np.float32(clip))
        w = np.clip(w_raw, -c, c)
        codes, s16, z16, s_pre, z_pre, t = quantize(w, shape.group)
        tq = np.nonzero(m_q)[0]
        pid = np.asarray(page_table)[seq_idx[tq], pos[tq] // PG].astype(np.int64)
        slot = pos[tq] % PG
        hh = np.arange(H)
        # per group g: fp16 s_g then z_g
        params = np.stack([s16, z16], -1).reshape(s16.shape[:-1] + (2 * s16.shape[-1],))
        pbytes = np.ascontiguousarray(params).view(np.uint16).astype("<u2").view(np.uint8).reshape(len(tq), H, pb)
        cache.pages[pid[:, None, None], hh[None, :, None],
                    (par_off + pb * slot)[:, None, None] + np.arange(pb)[None, None, :]] = pbytes
        if name == "K":
            kb = pack_k_codes(codes)                       # [Tq][H][32]
            cache.pages[pid[:, None, None], hh[None, :, None],
                        (codes_off + 32 * slot)[:, None, None] + np.arange(32)[None, None, :]] = kb
        else:
            # channel-major words: read-modify-write one slot value at a time so
            # tokens of one call sharing a page never overwrite each other.
            words = cache.pages[..., V_CODES:V_CODES + 512].copy().view("<u4")  # [N][H][128]
            for sv in np.unique(slot):
                sel = slot == sv
                p_ = pid[sel]
                old = words[p_]                                            # [n][H][128]
                mask = np.uint32(~np.uint32(3 << (2 * int(sv))) & 0xFFFFFFFF)
                new = (old & mask) | (codes[sel].astype(np.uint32) << np.uint32(2 * int(sv)))
                words[p_] = new
            cache.pages[..., V_CODES:V_CODES + 512] = words.view(np.uint8).reshape(
                cache.pages.shape[0], H, 512)
        info[name] = dict(token=tq, w=w, w_raw=w_raw, codes=codes, s16=s16, z16=z16,
                          s_pre=s_pre, z_pre=z_pre, t=t, page=pid, slot=slot)
    return info


# ----------------------------------------------------------------------------
# read path
# ----------------------------------------------------------------------------
def _dequant_rotated(shape: Shape, cache: Cache, h: int, pid, slot, which: str):
    """Rotated-basis reconstruction k_hat'_j = z_g + s_g * code_j (fp64) for the
    INT2 tokens at (pid, slot)."""
    blk = cache.pages[pid, h]                              # [n][block bytes]
    n = len(pid)
    _, k_par, v_par, pb = block_layout(shape.group)
    if which == "K":
        kb = blk[np.arange(n)[:, None], K_CODES + 32 * slot[:, None] + np.arange(32)[None, :]]
        codes = unpack_k_codes(kb)                         # [n][128]
        par = blk[np.arange(n)[:, None], k_par + pb * slot[:, None] + np.arange(pb)[None, :]]
    else:
        words = np.ascontiguousarray(blk[:, V_CODES:V_CODES + 512]).view("<u4")  # [n][128]
        codes = (words >> (2 * slot[:, None]).astype(np.uint32)) & 3
        par = blk[np.arange(n)[:, None], v_par + pb * slot[:, None] + np.arange(pb)[None, :]]
    par = np.ascontiguousarray(par).view("<f2").astype(np.float64)   # [n][2 per group]: s_g, z_g
    g = np.arange(D) // shape.group
    s = par[:, 0::2][:, g]
    z = par[:, 1::2][:, g]
    return z + s * codes.astype(np.float64)


def gather_sequence(shape: Shape, cache: Cache, layer: Layer, b: int, h: int,
                    L: int, page_table):
    """All L keys and values of sequence slot b, KV head h, in the original
    basis, fp64: BF16 regions read bit-exactly, INT2 history dequantized and
    inverse-rotated explicitly, k_hat = k_hat' R_K^T ([it] layout section: the
    read kernel unpacks, dequantizes and inverts the rotation; [es] 2.2 B).
    Returns (K [L][128], V [L][128], region labels [L])."""
    (s_lo, s_hi), (i_lo, i_hi), (r_lo, r_hi) = regions(L, shape.sink, shape.recent)
    K = np.zeros((L, D))
    V = np.zeros((L, D))
    lab = np.zeros(L, np.int8)
    if s_hi > s_lo:
        K[s_lo:s_hi] = bf16_to_f64(cache.k_sink[b, h, s_lo:s_hi])
        V[s_lo:s_hi] = bf16_to_f64(cache.v_sink[b, h, s_lo:s_hi])
        lab[s_lo:s_hi] = 0
    if i_hi > i_lo:
        p = np.arange(i_lo, i_hi)
        pid = np.asarray(page_table)[b, p // shape.page_size].astype(np.int64)
        slot = p % shape.page_size
        Rk = rotation(layer.u_k[h])
        Rv = rotation(layer.u_v[h])
        K[i_lo:i_hi] = _dequant_rotated(shape, cache, h, pid, slot, "K") @ Rk.T
        V[i_lo:i_hi] = _dequant_rotated(shape, cache, h, pid, slot, "V") @ Rv.T
        lab[i_lo:i_hi] = 1
    if r_hi > r_lo:
        p = np.arange(r_lo, r_hi)
        K[r_lo:r_hi] = bf16_to_f64(cache.k_ring[b, h, p % shape.recent])
        V[r_lo:r_hi] = bf16_to_f64(cache.v_ring[b, h, p % shape.recent])
        lab[r_lo:r_hi] = 2
    return K, V, lab


def decode(shape: Shape, cache: Cache, layer: Layer, q_bits, page_table, seq_lens,
           sm_scale: float, batches=None, heads=None):
    """Decode attention for one new query per sequence, fp64.

    out[b, hq] = softmax(sm_scale * q . K^T) V over the L = seq_lens[b] cached
    tokens of KV head hq // G.  L == 0 gives zeros.  ``batches``/``heads``
    restrict the computation to a sample (others are left at zero)."""
    q = bf16_to_f64(q_bits)
    B, Hq, _ = q.shape
    G = shape.gqa
    out = np.zeros((B, Hq, D))
    batches = range(B) if batches is None else batches
    kv_heads = range(shape.num_kv_heads) if heads is None else heads
    for b in batches:
        L = int(seq_lens[b])
        if L == 0:
            continue
        for h in kv_heads:
            K, V, _ = gather_sequence(shape, cache, layer, b, h, L, page_table)
            for hq in range(h * G, (h + 1) * G):
                logits = sm_scale * (K @ q[b, hq])
                p = np.exp(logits - logits.max())
                out[b, hq] = (p @ V) / p.sum()
    return out


def decode_folded(shape: Shape, cache: Cache, layer: Layer, q_bits, page_table,
                  seq_lens, sm_scale: float):
    """Self-check only: the same attention with the rotation folded onto the
    query (q' = q R_K) and the output (acc R_V^T), as the GPU path computes it.
    Equal to ``decode`` by associativity."""
    q = bf16_to_f64(q_bits)
    B, Hq, _ = q.shape
    G = shape.gqa
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        (s_lo, s_hi), (i_lo, i_hi), (r_lo, r_hi) = regions(L, shape.sink, shape.recent)
        for h in range(shape.num_kv_heads):
            Rk = rotation(layer.u_k[h])
            Rv = rotation(layer.u_v[h])
            plainK = np.concatenate([bf16_to_f64(cache.k_sink[b, h, s_lo:s_hi]),
                                     bf16_to_f64(cache.k_ring[b, h, np.arange(r_lo, r_hi) % shape.recent])])
            plainV = np.concatenate([bf16_to_f64(cache.v_sink[b, h, s_lo:s_hi]),
                                     bf16_to_f64(cache.v_ring[b, h, np.arange(r_lo, r_hi) % shape.recent])])
            p_ = np.arange(i_lo, i_hi)
            pid = np.asarray(page_table)[b, p_ // shape.page_size].astype(np.int64)
            slot = p_ % shape.page_size
            Kr = _dequant_rotated(shape, cache, h, pid, slot, "K")
            Vr = _dequant_rotated(shape, cache, h, pid, slot, "V")
            for hq in range(h * G, (h + 1) * G):
                qr = q[b, hq] @ Rk
                lg = np.concatenate([sm_scale * (plainK @ q[b, hq]), sm_scale * (Kr @ qr)])
                p = np.exp(lg - lg.max())
                npl = len(plainK)
                acc = p[:npl] @ plainV + (p[npl:] @ Vr) @ Rv.T
                out[b, hq] = acc / p.sum()
    return out


def extend(shape: Shape, cache: Cache, layer: Layer, q_bits, k_bits, v_bits, cu_seqlens,
           prefix_lens, page_table, sm_scale: float):
    """Chunked-prefill (extend) attention over the mixed cache, fp64.

    The read path of the Italian page's section "Architettura del Sistema di
    Serving e Layout di Memoria" and of the Spanish summary's 2.2 B (paged
    attention over the mixed cache, prefix caching) for a chunk of new tokens
    instead of one.  Reading taken where the pages are silent: the chunk of
    sequence slot b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of q (bf16
    [T][Hq][128]) and of k, v (bf16 [T][H_kv][128]); its i-th token sits at
    position prefix_lens[b] + i and attends to
      - the cached prefix [0, L_prev), L_prev = prefix_lens[b], as the cache
        stores it for a sequence of that length (gather_sequence: sink and
        ring rows exact, INT2 history dequantized and inverse-rotated), and
      - the chunk's own keys 0..i, in BF16 as given (causal),
    with softmax(sm_scale q . k) over all of them.  The chunk is not in the
    cache yet (it is written afterwards).  Returns out [T][Hq][128]."""
    q = bf16_to_f64(q_bits)
    kn = bf16_to_f64(k_bits)
    vn = bf16_to_f64(v_bits)
    T, Hq, _ = q.shape
    G = shape.gqa
    out = np.zeros((T, Hq, D))
    cu = np.asarray(cu_seqlens, np.int64)
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        L = int(prefix_lens[b])
        for h in range(shape.num_kv_heads):
            Kp, Vp, _ = gather_sequence(shape, cache, layer, b, h, L, page_table)
            for t in range(t0, t1):
                K = np.concatenate([Kp, kn[t0:t + 1, h]])
                V = np.concatenate([Vp, vn[t0:t + 1, h]])
                for hq in range(h * G, (h + 1) * G):
                    logits = sm_scale * (K @ q[t, hq])
                    p = np.exp(logits - logits.max())
                    out[t, hq] = (p @ V) / p.sum()
    return out


# ----------------------------------------------------------------------------
# all-BF16 paged cache: the baseline OSCAR is measured against ([it] "Velocita
# di decodifica" and [es] section 4 state the 100K-context decode speedups
# relative to a BF16 KV cache).  Block per (physical page, KV head): 4096 bf16
# elements, K token-major (slot t, channel c at 128 t + c), then V
# channel-major (channel c, slot t at 2048 + 16 c + t).  The layout is this
# library's own; the pages only say the cache is paged.
# ----------------------------------------------------------------------------
BF16_BLOCK = 4096


def new_bf16_pages(num_pages: int, num_kv_heads: int) -> np.ndarray:
    return np.zeros((num_pages, num_kv_heads, BF16_BLOCK), np.uint16)


def bf16_pages_write(pages: np.ndarray, k_bits, v_bits, seq_idx, pos, page_table,
                     page_size: int = 16) -> None:
    """Store tokens (bf16 bits [T][H][128]) unchanged: token (seq, pos) goes to
    slot pos % 16 of physical page page_table[seq][pos // 16]."""
    k_bits = np.asarray(k_bits, np.uint16)
    v_bits = np.asarray(v_bits, np.uint16)
    table = np.asarray(page_table)
    ch = np.arange(D)
    for t in range(len(seq_idx)):
        pid = int(table[int(seq_idx[t]), int(pos[t]) // page_size])
        slot = int(pos[t]) % page_size
        blk = pages[pid]                        # [H][4096] view
        blk[:, D * slot + ch] = k_bits[t]
        blk[:, 2048 + 16 * ch + slot] = v_bits[t]


def bf16_pages_gather(pages: np.ndarray, page_table, b: int, h: int, L: int, page_size: int = 16):
    """K and V [L][128] (fp64, exact) of sequence b, KV head h from the BF16 pages."""
    p = np.arange(L)
    pid = np.asarray(page_table)[b, p // page_size].astype(np.int64)
    slot = (p % page_size)[:, None]
    ch = np.arange(D)[None, :]
    blocks = pages[pid, h]                      # [L][4096]
    K = np.take_along_axis(blocks, D * slot + ch, axis=1)
    V = np.take_along_axis(blocks, 2048 + 16 * ch + slot, axis=1)
    return bf16_to_f64(K), bf16_to_f64(V)


def decode_bf16_paged(pages: np.ndarray, q_bits, page_table, seq_lens, num_kv_heads: int,
                      sm_scale: float, batches=None, heads=None):
    """Plain decode attention over the all-BF16 paged cache, fp64:
    out[b, hq] = softmax(sm_scale * q . K^T) V over the L = seq_lens[b] tokens
    of KV head hq // G.  L == 0 gives zeros.  ``batches``/``heads`` restrict the
    computation to a sample (others are left at zero)."""
    q = bf16_to_f64(q_bits)
    B, Hq, _ = q.shape
    G = Hq // num_kv_heads
    out = np.zeros((B, Hq, D))
    batches = range(B) if batches is None else batches
    kv_heads = range(num_kv_heads) if heads is None else heads
    for b in batches:
        L = int(seq_lens[b])
        if L == 0:
            continue
        for h in kv_heads:
            K, V = bf16_pages_gather(pages, page_table, b, h, L)
            for hq in range(h * G, (h + 1) * G):
                logits = sm_scale * (K @ q[b, hq])
                p = np.exp(logits - logits.max())
                out[b, hq] = (p @ V) / p.sum()
    return out


# ----------------------------------------------------------------------------
# offline calibration ([es] 2.2 A "Fase de Calibracion Offline"; [ru] paragraph 2)
# ----------------------------------------------------------------------------
def query_covariance(q_cal_h: np.ndarray) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n^T q_n over the N calibration queries of the G query
    heads that share one KV head (pooled: N = G * n_samples)."""
    Q = q_cal_h.reshape(-1, q_cal_h.shape[-1])
    return Q.T @ Q / Q.shape[0]


def score_weighted_covariance(q_cal_h, k_cal_h, v_cal_h, sm_scale: float) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V with S the causal softmax attention of each query
    head over the calibration keys, pooled over the G heads ([ru] paragraph 2,
    [es] 2.1 and 2.2 A.1).  Reading: S is the post-softmax probability matrix
    with a causal mask, so S V is the attention output."""
    G, N, d = q_cal_h.shape
    C = np.zeros((d, d))
    causal = np.tril(np.ones((N, N), bool))
    for g in range(G):
        lg = sm_scale * (q_cal_h[g] @ k_cal_h.T)
        lg = np.where(causal, lg, -np.inf)
        lg -= lg.max(axis=1, keepdims=True)
        S = np.exp(lg)
        S /= S.sum(axis=1, keepdims=True)
        O = S @ v_cal_h
        C += O.T @ O
    return C / (G * N)


def eigenbasis(C: np.ndarray):
    """Eigenvectors of a symmetric matrix as columns, eigenvalues descending,
    each column signed so its largest-magnitude entry (first on ties) is
    positive.  Returns (U, eigenvalues)."""
    lam, U = np.linalg.eigh(C)
    order = np.argsort(-lam, kind="stable")
    lam, U = lam[order], U[:, order]
    idx = np.argmax(np.abs(U), axis=0)
    sign = np.sign(U[idx, np.arange(U.shape[1])])
    sign[sign == 0] = 1.0
    return U * sign, lam


def calibrate_layer(q_cal, k_cal, v_cal, sm_scale: float, quantile: float = 0.999):
    """Offline calibration of one layer ([es] 2.2 A steps 1-4).

    q_cal [H][G][N][128], k_cal/v_cal [H][N][128] (float64).  Per KV head:
    U_Q = eigenbasis(C_Q), U_S = eigenbasis(C_S), rounded to bf16 (the form the
    kernels consume).  Per layer: clip_K / clip_V = the 0.999 quantile (linear
    interpolation) of |rotated calibration values| over all heads, tokens and
    channels, rotated with the bf16 U; stored as float32."""
    H = k_cal.shape[0]
    uq64, us64, uk_bits, uv_bits = [], [], [], []
    for h in range(H):
        Uq, _ = eigenbasis(query_covariance(q_cal[h]))
        Us, _ = eigenbasis(score_weighted_covariance(q_cal[h], k_cal[h], v_cal[h], sm_scale))
        uq64.append(Uq)
        us64.append(Us)
        uk_bits.append(f64_to_bf16(Uq))
        uv_bits.append(f64_to_bf16(Us))
    uk_bits = np.stack(uk_bits)
    uv_bits = np.stack(uv_bits)
    rk = np.concatenate([np.abs(k_cal[h] @ rotation(uk_bits[h])).ravel() for h in range(H)])
    rv = np.concatenate([np.abs(v_cal[h] @ rotation(uv_bits[h])).ravel() for h in range(H)])
    clip_k = np.float32(np.quantile(rk, quantile))
    clip_v = np.float32(np.quantile(rv, quantile))
    return dict(u_k=uk_bits, u_v=uv_bits, clip_k=clip_k, clip_v=clip_v,
                U_Q=np.stack(uq64), U_S=np.stack(us64))
