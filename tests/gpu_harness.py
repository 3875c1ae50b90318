"""Shared machinery of the GPU parity tests: move caches between the oracle
(NumPy) and the library (torch device memory), and compare them.

Parity rules (written out here, used by every GPU test):
  * page bytes, sink rows and ring rows are compared bit for bit;
  * an INT2 code may differ only where the oracle's pre-rounding value t lies
    within 1e-5 relative of a decision boundary b in {0.5, 1.5, 2.5};
  * an fp16 scale or zero may differ only where its fp64 pre-rounding value
    lies within 1e-5 (relative to max(|value|, scale)) of an fp16 rounding
    midpoint; the codes of such a group are then re-derived by the oracle's
    rule with the GPU's scale and zero and held to the rule above;
  * "relative" is taken relative to the operands the kernel's fp32 arithmetic
    works on, not only to the result: the rotated values of a token carry an
    fp32 error that scales with the token's largest rotated magnitude, so
    each window is at least that allowance, E_w = 8 fp32 ulps of
    max_j |w_raw_j| (2^-21 max|w_raw|): scale 2/3 E_w, zero E_w, code t
    4 E_w / s.  This only matters for ill-conditioned groups whose range is
    tiny next to their values (e.g. 64 values clipped at or just below c:
    range 3.5e-3 at magnitude 18.7, where fp32 alone moves s by 1e-3
    relative); elsewhere 1e-5 relative is the wider window.  Such excusals
    are counted separately (codes_cond, params_cond) and may not exceed 1e-4
    of the codes / parameters a call writes;
  * bytes outside the slots a call writes must be untouched;
  * decode outputs are bf16; "in bf16 units" is read as: the error of an
    element beyond its own bf16 representation error,
    e = max(0, |out_gpu - out_ref| - ulp_bf16(out_ref) / 2), must satisfy
    max e <= 2e-2 and mean e <= 2e-3 (an absolute 2e-2 is below bf16's own
    resolution once |out| > 8, e.g. V outlier channels x20).
"""
from __future__ import annotations

import math

import numpy as np

import oracle as O

SIG = 1 / math.sqrt(128)
CODE_REL_TOL = 1e-5
W_ULP_ALLOWANCE = 2.0 ** -21   # 8 fp32 ulps of the token's largest rotated magnitude
COND_FRACTION = 1e-4           # at most this share of codes / parameters excused by that allowance alone
MAX_ABS_TOL = 2e-2
MEAN_ABS_TOL = 2e-3


def to_dev_bf16(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def from_dev_bf16(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_i32(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to(device)


def device_cache(shape: O.Shape, cache: O.Cache, layer: O.Layer, device):
    """Library cache buffers holding a copy of an oracle cache."""
    import torch
    import int2_rotated_kv_write_amd as lib
    return lib.CacheBuffers(
        pages=torch.from_numpy(cache.pages.copy()).to(device),
        k_sink=to_dev_bf16(cache.k_sink, device), v_sink=to_dev_bf16(cache.v_sink, device),
        k_ring=to_dev_bf16(cache.k_ring, device), v_ring=to_dev_bf16(cache.v_ring, device),
        u_k=to_dev_bf16(layer.u_k, device), u_v=to_dev_bf16(layer.u_v, device),
        clip_k=float(layer.clip_k), clip_v=float(layer.clip_v))


def lib_shape(shape: O.Shape):
    import int2_rotated_kv_write_amd as lib
    return lib.CacheShape(shape.num_kv_heads, shape.num_q_heads, 128, shape.page_size,
                          shape.sink, shape.recent, shape.group)


def host_cache(dc) -> O.Cache:
    return O.Cache(pages=dc.pages.cpu().numpy(), k_sink=from_dev_bf16(dc.k_sink),
                   v_sink=from_dev_bf16(dc.v_sink), k_ring=from_dev_bf16(dc.k_ring),
                   v_ring=from_dev_bf16(dc.v_ring))


def _near_fp16_midpoint(x, scale, slack=0.0):
    d = np.maximum(CODE_REL_TOL * np.maximum(np.abs(x), np.abs(scale)), slack)
    return O.fp16_rne(x - d).view(np.uint16) != O.fp16_rne(x + d).view(np.uint16)


def _near_code_boundary(t, slack=0.0):
    near = np.zeros(t.shape, bool)
    for b in (0.5, 1.5, 2.5):
        near |= np.abs(t - b) <= np.maximum(CODE_REL_TOL * b, slack)
    return near


def _gpu_codes(pages, kind, pid, h, slot, group=64):
    n = len(pid)
    hh = np.broadcast_to(h, (n,))
    blk = pages[pid, hh]                                   # [n][block bytes]
    _, k_par, v_par, pb = O.block_layout(group)
    if kind == "K":
        kb = blk[np.arange(n)[:, None], O.K_CODES + 32 * slot[:, None] + np.arange(32)[None, :]]
        codes = O.unpack_k_codes(kb)
        par = blk[np.arange(n)[:, None], k_par + pb * slot[:, None] + np.arange(pb)[None, :]]
    else:
        words = np.ascontiguousarray(blk[:, O.V_CODES:O.V_CODES + 512]).view("<u4")
        codes = ((words >> (2 * slot[:, None]).astype(np.uint32)) & 3).astype(np.uint8)
        par = blk[np.arange(n)[:, None], v_par + pb * slot[:, None] + np.arange(pb)[None, :]]
    return codes, np.ascontiguousarray(par).view("<u2")     # [n][128], [n][2 per group]: s_g, z_g


def compare_kv_write(shape: O.Shape, ref: O.Cache, got: O.Cache, info: dict, got_before: O.Cache):
    """Assert GPU-written cache `got` matches the oracle's `ref` under the
    parity rules; `info` is the oracle's kv_write diagnostics of this call and
    `got_before` the GPU cache before it (bytes the call must not touch are
    compared against it: earlier calls may differ from the oracle by excused
    near-ties).  Returns counts of excused codes / parameters."""
    stats = dict(codes=0, codes_excused=0, codes_cond=0, params=0, params_excused=0, params_cond=0)
    H = shape.num_kv_heads
    _, k_par, v_par, pb = O.block_layout(shape.group)
    assert np.array_equal(ref.k_sink, got.k_sink), "k_sink differs"
    assert np.array_equal(ref.v_sink, got.v_sink), "v_sink differs"
    assert np.array_equal(ref.k_ring, got.k_ring), "k_ring differs"
    assert np.array_equal(ref.v_ring, got.v_ring), "v_ring differs"
    touched = np.zeros(ref.pages.shape, bool)
    for kind, d in info.items():
        pid, slot = d["page"], d["slot"]
        for h in range(H):
            codes, par = _gpu_codes(got.pages, kind, pid, h, slot, shape.group)
            s_ref = d["s16"][:, h].view(np.uint16)              # [n][2]
            z_ref = d["z16"][:, h].view(np.uint16)
            s_got, z_got = par[:, 0::2], par[:, 1::2]
            s_pre, z_pre = d["s_pre"][:, h], d["z_pre"][:, h]
            e_w = W_ULP_ALLOWANCE * np.abs(d["w_raw"][:, h]).max(axis=1)[:, None]   # [n][1]
            near_s = _near_fp16_midpoint(s_pre, s_pre, 2.0 / 3.0 * e_w)
            near_z = _near_fp16_midpoint(z_pre, s_pre, e_w)
            bad_s = (s_got != s_ref) & ~near_s
            bad_z = (z_got != z_ref) & ~near_z
            stats["params_cond"] += int((((s_got != s_ref) & ~_near_fp16_midpoint(s_pre, s_pre))
                                         | ((z_got != z_ref) & ~_near_fp16_midpoint(z_pre, s_pre))).sum())
            for bad, what in ((bad_s, "scale"), (bad_z, "zero")):
                if bad.any():
                    i, g = np.argwhere(bad)[0]
                    seg = d["w"][i, h, shape.group * g:shape.group * (g + 1)]
                    raise AssertionError(
                        f"{kind} {what} mismatch h={h} at token {i} group {g} ({int(bad.sum())} total): "
                        f"s_pre={s_pre[i, g]!r} z_pre={z_pre[i, g]!r} ref s,z=0x{s_ref[i, g]:04x},0x{z_ref[i, g]:04x} "
                        f"gpu s,z=0x{s_got[i, g]:04x},0x{z_got[i, g]:04x} group max={seg.max()!r} min={seg.min()!r} "
                        f"max|w_raw|={np.abs(d['w_raw'][i, h]).max()!r}")
            stats["params"] += s_ref.size * 2
            stats["params_excused"] += int((s_got != s_ref).sum() + (z_got != z_ref).sum())
            # reference codes, re-derived with the GPU's parameters where they differ
            w = d["w"][:, h]                                      # [n][128]
            g = np.arange(128) // shape.group
            sg = s_got.view(np.float16).astype(np.float64)[:, g]
            zg = z_got.view(np.float16).astype(np.float64)[:, g]
            t = np.where(sg == 0, 0.0, (w - zg) / np.where(sg == 0, 1.0, sg))
            code_ref = np.where(sg == 0, 0, np.clip(np.rint(t), 0, 3)).astype(np.uint8)
            same = (s_got == s_ref) & (z_got == z_ref)
            assert np.array_equal(code_ref[same[:, g]], d["codes"][:, h][same[:, g]])
            mism = codes != code_ref
            slack = np.where(sg == 0, 0.0, 4.0 * e_w / np.where(sg == 0, 1.0, sg))
            bad = mism & ~_near_code_boundary(t, slack)
            stats["codes_cond"] += int((mism & ~_near_code_boundary(t)).sum())
            if bad.any():
                i, c = np.argwhere(bad)[0]
                gg = c // shape.group
                raise AssertionError(
                    f"{kind} code mismatch h={h}: {int(bad.sum())} codes, e.g. t={t[bad][:4]}, gpu={codes[bad][:4]}, "
                    f"ref={code_ref[bad][:4]}; token {i} group {gg}: gpu s,z=0x{s_got[i, gg]:04x},0x{z_got[i, gg]:04x} "
                    f"ref s,z=0x{s_ref[i, gg]:04x},0x{z_ref[i, gg]:04x} w[min,max]=({w[i].min()!r},{w[i].max()!r}) "
                    f"max|w_raw|={np.abs(d['w_raw'][i, h]).max()!r}")
            stats["codes"] += codes.size
            stats["codes_excused"] += int(mism.sum())
            # bytes this call may have written
            hh = np.full(len(pid), h)
            if kind == "K":
                cols = O.K_CODES + 32 * slot[:, None] + np.arange(32)[None, :]
                touched[pid[:, None], hh[:, None], cols] = True
                cols = k_par + pb * slot[:, None] + np.arange(pb)[None, :]
            else:
                touched[pid[:, None], hh[:, None], O.V_CODES + np.arange(512)[None, :]] = True
                cols = v_par + pb * slot[:, None] + np.arange(pb)[None, :]
            touched[pid[:, None], hh[:, None], cols] = True
    # V words: bits of slots not written by this call must be unchanged
    base = got_before.pages
    wr = np.ascontiguousarray(got.pages[..., O.V_CODES:O.V_CODES + 512]).view("<u4")
    wb = np.ascontiguousarray(base[..., O.V_CODES:O.V_CODES + 512]).view("<u4")
    keep = np.full(wr.shape, 0xFFFFFFFF, np.uint32)
    if "V" in info:
        d = info["V"]
        for h in range(H):
            for sl in np.unique(d["slot"]):
                sel = d["slot"] == sl
                keep[d["page"][sel], h, :] &= np.uint32(~np.uint32(3 << (2 * int(sl))) & 0xFFFFFFFF)
    assert np.array_equal(wr & keep, wb & keep), "V code bits of unwritten slots changed"
    assert np.array_equal(got.pages[~touched], base[~touched]), "bytes outside written slots changed"
    # the operand-magnitude allowance may excuse only a rare ill-conditioned group: a
    # systematic fp32 error of that size would show up here as a large count
    assert stats["codes_cond"] <= math.ceil(COND_FRACTION * stats["codes"]), stats
    assert stats["params_cond"] <= math.ceil(COND_FRACTION * stats["params"]), stats
    return stats


def ulp_bf16(x):
    """Spacing of bf16 values at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def compare_outputs(out_gpu_bits: np.ndarray, out_ref: np.ndarray, sel=None):
    got = O.bf16_to_f64(out_gpu_bits)
    if sel is not None:
        got, out_ref = got[sel], out_ref[sel]
    assert np.isfinite(got).all(), "non-finite GPU output"
    raw = np.abs(got - out_ref)
    err = np.maximum(0.0, raw - ulp_bf16(out_ref) / 2)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS_TOL, f"max error beyond bf16 rounding {mx} (raw {raw.max()})"
    assert mean <= MEAN_ABS_TOL, f"mean error beyond bf16 rounding {mean} (raw {raw.mean()})"
    return dict(max=mx, mean=mean, raw_max=float(raw.max()), raw_mean=float(raw.mean()))
