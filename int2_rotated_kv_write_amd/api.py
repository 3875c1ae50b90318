"""Python face of the C ABI: argument marshalling only.

Every function checks tensor dtypes, devices and shapes, passes raw pointers
and the current HIP stream to the library, and raises OscarError on a
non-zero status.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import numpy as np

from ._native import OscarLayer, OscarShape, load

HEAD_DIM = 128
PAGE_BLOCK = 1280          # page block bytes with 64-channel groups
PAGE_BLOCK_G128 = 1152     # ... with one 128-channel group per token
BF16_PAGE_ELEMS = 4096     # bf16 elements per (page, KV head) of the BF16 baseline cache


class OscarError(RuntimeError):
    pass


def status_string(code: int) -> str:
    return load().oscar_status_string(code).decode()


def _check(rc: int):
    if rc != 0:
        lib = load()
        raise OscarError(f"{lib.oscar_status_string(rc).decode()} ({rc}): {lib.oscar_last_error().decode()}")


@dataclass(frozen=True)
class CacheShape:
    num_kv_heads: int
    num_q_heads: int
    head_dim: int = HEAD_DIM
    page_size: int = 16
    sink: int = 64
    recent: int = 256
    group: int = 64

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def block_bytes(self) -> int:
        return PAGE_BLOCK_G128 if self.group == 128 else PAGE_BLOCK

    def c(self) -> OscarShape:
        return OscarShape(self.num_kv_heads, self.num_q_heads, self.head_dim, self.page_size,
                          self.sink, self.recent, self.group)


@dataclass
class CacheBuffers:
    """One layer's device buffers (layouts in include/oscar.h)."""
    pages: "torch.Tensor"      # uint8 [num_pages][H_kv][1280, or 1152 with 128-channel groups]
    k_sink: "torch.Tensor"     # bfloat16 [slots][H_kv][sink][128]
    v_sink: "torch.Tensor"
    k_ring: "torch.Tensor"     # bfloat16 [slots][H_kv][recent][128]
    v_ring: "torch.Tensor"
    u_k: "torch.Tensor"        # bfloat16 [H_kv][128][128]
    u_v: "torch.Tensor"
    clip_k: float
    clip_v: float

    def c(self) -> OscarLayer:
        return OscarLayer(self.pages.data_ptr(), self.k_sink.data_ptr(), self.v_sink.data_ptr(),
                          self.k_ring.data_ptr(), self.v_ring.data_ptr(), self.u_k.data_ptr(),
                          self.u_v.data_ptr(), float(self.clip_k), float(self.clip_v))


def allocate_cache(shape: CacheShape, num_pages: int, num_slots: int, device,
                   u_k=None, u_v=None, clip_k: float = 1.0, clip_v: float = 1.0) -> CacheBuffers:
    import torch
    H = shape.num_kv_heads
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device=device)
    if u_k is None:
        u_k = z(H, HEAD_DIM, HEAD_DIM)
    if u_v is None:
        u_v = z(H, HEAD_DIM, HEAD_DIM)
    return CacheBuffers(
        pages=z(num_pages, H, shape.block_bytes, dt=torch.uint8),
        k_sink=z(num_slots, H, max(shape.sink, 1), HEAD_DIM),
        v_sink=z(num_slots, H, max(shape.sink, 1), HEAD_DIM),
        k_ring=z(num_slots, H, shape.recent, HEAD_DIM),
        v_ring=z(num_slots, H, shape.recent, HEAD_DIM),
        u_k=u_k, u_v=u_v, clip_k=clip_k, clip_v=clip_v)


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t, dtype, name, shape=None):
    import torch
    if t is None:
        return None
    if not t.is_cuda:
        raise OscarError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise OscarError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise OscarError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise OscarError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    align = 4 if dtype == torch.int32 else 16     # the alignment rules of include/oscar.h
    if t.data_ptr() % align:
        raise OscarError(f"{name} must start on a {align}-byte boundary")
    return t.data_ptr()


def _check_cache(shape: CacheShape, cache: CacheBuffers):
    import torch
    H = shape.num_kv_heads
    if cache.pages.dim() != 3 or cache.pages.shape[1:] != (H, shape.block_bytes):
        raise OscarError(f"pages must be [num_pages][H_kv][{shape.block_bytes}]")
    _dev(cache.pages, torch.uint8, "pages")
    for n in ("k_sink", "v_sink", "k_ring", "v_ring"):
        _dev(getattr(cache, n), torch.bfloat16, n)
    for n in ("u_k", "u_v"):
        _dev(getattr(cache, n), torch.bfloat16, n, (H, HEAD_DIM, HEAD_DIM))


def kv_write(shape: CacheShape, cache: CacheBuffers, k, v, seq_idx, pos, page_table,
             seq_lens_after, stream=None) -> None:
    """oscar_kv_write: rotate, clip, quantize and pack tokens (k and/or v:
    bfloat16 [T][H_kv][128]) into the cache."""
    import torch
    _check_cache(shape, cache)
    T = int(seq_idx.numel())
    H = shape.num_kv_heads
    kp = _dev(k, torch.bfloat16, "k", (T, H, HEAD_DIM))
    vp = _dev(v, torch.bfloat16, "v", (T, H, HEAD_DIM))
    if page_table.dim() != 2:
        raise OscarError("page_table must be [num_slots][max_pages]")
    rc = load().oscar_kv_write(
        ctypes.byref(shape.c()), ctypes.byref(cache.c()), kp, vp,
        _dev(seq_idx, torch.int32, "seq_idx", (T,)), _dev(pos, torch.int32, "pos", (T,)), T,
        _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
        _dev(seq_lens_after, torch.int32, "seq_lens_after"), _stream(stream))
    _check(rc)


def decode_workspace_bytes(shape: CacheShape, batch: int, max_pages: int) -> int:
    return int(load().oscar_decode_workspace_bytes(ctypes.byref(shape.c()), batch, max_pages))


def decode_attn(shape: CacheShape, cache: CacheBuffers, q, page_table, seq_lens, out, workspace,
                sm_scale: float | None = None, stream=None) -> None:
    """oscar_decode_attn: out (bfloat16 [B][Hq][128]) = attention of q over the
    cache for sequence lengths seq_lens (int32 [B])."""
    import torch
    _check_cache(shape, cache)
    B = int(seq_lens.numel())
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if page_table.dim() != 2 or page_table.shape[0] < B:
        raise OscarError("page_table must be [>= batch][max_pages]")
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise OscarError("workspace must be a uint8 device tensor")
    rc = load().oscar_decode_attn(
        ctypes.byref(shape.c()), ctypes.byref(cache.c()),
        _dev(q, torch.bfloat16, "q", (B, shape.num_q_heads, HEAD_DIM)),
        _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens", (B,)), B, float(sm_scale),
        _dev(out, torch.bfloat16, "out", (B, shape.num_q_heads, HEAD_DIM)),
        workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(rc)


def cascade_workspace_bytes(shape: CacheShape, batch: int, max_pages: int, max_shared_pages: int) -> int:
    return int(load().oscar_cascade_workspace_bytes(ctypes.byref(shape.c()), batch, max_pages, max_shared_pages))


def _cascade_args(shape, cache, q, page_table, seq_lens, cu_groups, group_pages, out, workspace, max_group,
                  max_shared_pages, sm_scale, stream):
    import torch
    _check_cache(shape, cache)
    B = int(seq_lens.numel())
    n_groups = int(group_pages.numel())
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if page_table.dim() != 2 or page_table.shape[0] < B:
        raise OscarError("page_table must be [>= batch][max_pages]")
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise OscarError("workspace must be a uint8 device tensor")
    cs, cl = shape.c(), cache.c()
    args = (ctypes.byref(cs), ctypes.byref(cl), _dev(q, torch.bfloat16, "q", (B, shape.num_q_heads, HEAD_DIM)),
            _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
            _dev(seq_lens, torch.int32, "seq_lens", (B,)), B,
            _dev(cu_groups, torch.int32, "cu_groups", (n_groups + 1,)), _dev(group_pages, torch.int32, "group_pages"),
            n_groups, int(max_group), int(max_shared_pages), float(sm_scale),
            _dev(out, torch.bfloat16, "out", (B, shape.num_q_heads, HEAD_DIM)),
            workspace.data_ptr(), workspace.numel(), _stream(stream))
    return args, (cs, cl, q, page_table, seq_lens, cu_groups, group_pages, out, workspace)


def decode_attn_cascade(shape: CacheShape, cache: CacheBuffers, q, page_table, seq_lens, cu_groups, group_pages,
                        out, workspace, max_group: int, max_shared_pages: int, sm_scale: float | None = None,
                        stream=None) -> None:
    """oscar_decode_attn_cascade: decode_attn where groups of sequences (batch
    entries cu_groups[g] .. cu_groups[g+1]-1, int32 [n_groups+1]) share their first
    group_pages[g] (int32 [n_groups]) INT2 pages; those pages are read once per
    block of the members' query heads.  Same result as decode_attn."""
    args, _ = _cascade_args(shape, cache, q, page_table, seq_lens, cu_groups, group_pages, out, workspace,
                            max_group, max_shared_pages, sm_scale, stream)
    _check(load().oscar_decode_attn_cascade(*args))


def prepare_decode_attn_cascade(shape: CacheShape, cache: CacheBuffers, q, page_table, seq_lens, cu_groups,
                                group_pages, out, workspace, max_group: int, max_shared_pages: int,
                                sm_scale: float | None = None, stream=None) -> PreparedCall:
    args, keep = _cascade_args(shape, cache, q, page_table, seq_lens, cu_groups, group_pages, out, workspace,
                               max_group, max_shared_pages, sm_scale, stream)
    return PreparedCall(load().oscar_decode_attn_cascade, args, keep)


def decode_attn_noalloc(shape: CacheShape, cache: CacheBuffers, q, page_table, seq_lens, out,
                        sm_scale: float | None = None, stream=None) -> None:
    """oscar_decode_attn_noalloc: decode_attn with the library's static device
    scratch instead of a workspace (no allocation anywhere; calls that overlap on
    one GPU race)."""
    import torch
    _check_cache(shape, cache)
    B = int(seq_lens.numel())
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if page_table.dim() != 2 or page_table.shape[0] < B:
        raise OscarError("page_table must be [>= batch][max_pages]")
    rc = load().oscar_decode_attn_noalloc(
        ctypes.byref(shape.c()), ctypes.byref(cache.c()),
        _dev(q, torch.bfloat16, "q", (B, shape.num_q_heads, HEAD_DIM)),
        _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens", (B,)), B, float(sm_scale),
        _dev(out, torch.bfloat16, "out", (B, shape.num_q_heads, HEAD_DIM)), _stream(stream))
    _check(rc)


def extend_workspace_bytes(shape: CacheShape, num_tokens: int, max_pages: int, max_chunk: int) -> int:
    return int(load().oscar_extend_workspace_bytes(ctypes.byref(shape.c()), num_tokens, max_pages, max_chunk))


def extend_attn(shape: CacheShape, cache: CacheBuffers, q, k, v, cu_seqlens, prefix_lens, page_table, out,
                workspace, max_chunk: int, sm_scale: float | None = None, stream=None) -> None:
    """oscar_extend_attn: chunked-prefill attention.  q (bfloat16 [T][Hq][128]) of the chunk
    tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 (int32 [B+1]) attends to the cached prefix of
    prefix_lens[b] (int32 [B]) tokens as stored and causally to the chunk's own k, v
    (bfloat16 [T][H_kv][128]); out bfloat16 [T][Hq][128].  The chunk is not yet in the
    cache: write it with kv_write afterwards."""
    import torch
    _check_cache(shape, cache)
    T = int(q.shape[0]) if q is not None else 0
    B = int(prefix_lens.numel())
    H = shape.num_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if page_table.dim() != 2 or page_table.shape[0] < B:
        raise OscarError("page_table must be [>= batch][max_pages]")
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise OscarError("workspace must be a uint8 device tensor")
    rc = load().oscar_extend_attn(
        ctypes.byref(shape.c()), ctypes.byref(cache.c()),
        _dev(q, torch.bfloat16, "q", (T, shape.num_q_heads, HEAD_DIM)),
        _dev(k, torch.bfloat16, "k", (T, H, HEAD_DIM)), _dev(v, torch.bfloat16, "v", (T, H, HEAD_DIM)),
        _dev(cu_seqlens, torch.int32, "cu_seqlens", (B + 1,)), _dev(prefix_lens, torch.int32, "prefix_lens", (B,)),
        B, T, int(max_chunk), _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
        float(sm_scale), _dev(out, torch.bfloat16, "out", (T, shape.num_q_heads, HEAD_DIM)),
        workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(rc)


def bf16_decode_workspace_bytes(num_kv_heads: int, num_q_heads: int, batch: int, max_pages: int) -> int:
    return int(load().oscar_bf16_decode_workspace_bytes(num_kv_heads, num_q_heads, batch, max_pages))


def _bf16_decode_args(num_kv_heads, num_q_heads, pages, q, page_table, seq_lens, out, workspace,
                      sm_scale, stream):
    import torch
    B = int(seq_lens.numel())
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if pages.dim() != 3 or tuple(pages.shape[1:]) != (num_kv_heads, BF16_PAGE_ELEMS):
        raise OscarError("pages must be bfloat16 [num_pages][H_kv][4096]")
    if page_table.dim() != 2 or page_table.shape[0] < B:
        raise OscarError("page_table must be [>= batch][max_pages]")
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise OscarError("workspace must be a uint8 device tensor")
    return (num_kv_heads, num_q_heads, _dev(pages, torch.bfloat16, "pages"),
            _dev(q, torch.bfloat16, "q", (B, num_q_heads, HEAD_DIM)),
            _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
            _dev(seq_lens, torch.int32, "seq_lens", (B,)), B, float(sm_scale),
            _dev(out, torch.bfloat16, "out", (B, num_q_heads, HEAD_DIM)),
            workspace.data_ptr(), workspace.numel(), _stream(stream))


def bf16_decode_attn(num_kv_heads: int, num_q_heads: int, pages, q, page_table, seq_lens, out, workspace,
                     sm_scale: float | None = None, stream=None) -> None:
    """oscar_bf16_decode_attn: the BF16 paged-cache baseline.  pages bfloat16
    [num_pages][H_kv][4096] (K token-major, then V channel-major per block),
    q / out bfloat16 [B][Hq][128], seq_lens int32 [B]."""
    _check(load().oscar_bf16_decode_attn(*_bf16_decode_args(num_kv_heads, num_q_heads, pages, q, page_table,
                                                            seq_lens, out, workspace, sm_scale, stream)))


def _decode_step_args(shape: CacheShape, cache: CacheBuffers, k, v, seq_idx, pos, seq_lens_after, q, page_table,
                      seq_lens, out, workspace, sm_scale, stream):
    import torch
    _check_cache(shape, cache)
    T = int(seq_idx.numel())
    H = shape.num_kv_heads
    B = int(seq_lens.numel())
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if page_table.dim() != 2:
        raise OscarError("page_table must be [num_slots][max_pages]")
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise OscarError("workspace must be a uint8 device tensor")
    cs, cl = shape.c(), cache.c()
    args = (ctypes.byref(cs), ctypes.byref(cl),
            _dev(k, torch.bfloat16, "k", (T, H, HEAD_DIM)), _dev(v, torch.bfloat16, "v", (T, H, HEAD_DIM)),
            _dev(seq_idx, torch.int32, "seq_idx", (T,)), _dev(pos, torch.int32, "pos", (T,)), T,
            _dev(seq_lens_after, torch.int32, "seq_lens_after"),
            _dev(q, torch.bfloat16, "q", (B, shape.num_q_heads, HEAD_DIM)),
            _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
            _dev(seq_lens, torch.int32, "seq_lens", (B,)), B, float(sm_scale),
            _dev(out, torch.bfloat16, "out", (B, shape.num_q_heads, HEAD_DIM)),
            workspace.data_ptr(), workspace.numel(), _stream(stream))
    return args, (cs, cl, k, v, seq_idx, pos, seq_lens_after, q, page_table, seq_lens, out, workspace)


def decode_step(shape: CacheShape, cache: CacheBuffers, k, v, seq_idx, pos, seq_lens_after, q, page_table,
                seq_lens, out, workspace, sm_scale: float | None = None, stream=None) -> None:
    """oscar_decode_step: kv_write of the new tokens (k, v bfloat16 [T][H_kv][128]
    at (seq_idx, pos)), then decode_attn of q (bfloat16 [B][Hq][128]) over
    seq_lens, in one call."""
    args, _keep = _decode_step_args(shape, cache, k, v, seq_idx, pos, seq_lens_after, q, page_table, seq_lens,
                                    out, workspace, sm_scale, stream)
    _check(load().oscar_decode_step(*args))


def calibrate_layer(q_cal: np.ndarray, k_cal: np.ndarray, v_cal: np.ndarray, sm_scale: float,
                    quantile: float = 0.999, num_threads: int = 0):
    """oscar_calibrate_layer (host, offline).  q_cal float64 [H][G][N][128],
    k_cal / v_cal float64 [H][N][128].  Returns (u_k, u_v) as uint16 bf16 bits
    [H][128][128] and (clip_k, clip_v) as float32."""
    q_cal = np.ascontiguousarray(q_cal, np.float64)
    k_cal = np.ascontiguousarray(k_cal, np.float64)
    v_cal = np.ascontiguousarray(v_cal, np.float64)
    H, G, N, D = q_cal.shape
    if D != HEAD_DIM or k_cal.shape != (H, N, D) or v_cal.shape != (H, N, D):
        raise OscarError("calibration arrays: q [H][G][N][128], k/v [H][N][128]")
    u_k = np.zeros((H, D, D), np.uint16)
    u_v = np.zeros((H, D, D), np.uint16)
    ck, cv = ctypes.c_float(), ctypes.c_float()
    dp = ctypes.POINTER(ctypes.c_double)
    rc = load().oscar_calibrate_layer(
        H, G, N, q_cal.ctypes.data_as(dp), k_cal.ctypes.data_as(dp), v_cal.ctypes.data_as(dp),
        float(sm_scale), float(quantile), u_k.ctypes.data, u_v.ctypes.data,
        ctypes.byref(ck), ctypes.byref(cv), int(num_threads))
    _check(rc)
    return u_k, u_v, np.float32(ck.value), np.float32(cv.value)


def calibrate_clip(x_cal: np.ndarray, u: np.ndarray, quantile: float = 0.999) -> np.float32:
    """oscar_calibrate_clip (host, offline): the clip threshold for the rotation
    basis u (uint16 bf16 bits [H][128][128]) from calibration rows x_cal
    (float64 [H][N][128])."""
    x_cal = np.ascontiguousarray(x_cal, np.float64)
    u = np.ascontiguousarray(u, np.uint16)
    H, N, D = x_cal.shape
    if D != HEAD_DIM or u.shape != (H, D, D):
        raise OscarError("x_cal [H][N][128], u [H][128][128]")
    c = ctypes.c_float()
    rc = load().oscar_calibrate_clip(H, N, x_cal.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), u.ctypes.data,
                                     float(quantile), ctypes.byref(c))
    _check(rc)
    return np.float32(c.value)


class PreparedCall:
    """A library call with its ctypes arguments built once (for tight loops);
    calling it re-issues the same launch on the same stream."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        _check(self._fn(*self._args))


def prepare_kv_write(shape: CacheShape, cache: CacheBuffers, k, v, seq_idx, pos, page_table,
                     seq_lens_after, stream=None) -> PreparedCall:
    import torch
    _check_cache(shape, cache)
    T = int(seq_idx.numel())
    H = shape.num_kv_heads
    cs, cl = shape.c(), cache.c()
    args = (ctypes.byref(cs), ctypes.byref(cl),
            _dev(k, torch.bfloat16, "k", (T, H, HEAD_DIM)), _dev(v, torch.bfloat16, "v", (T, H, HEAD_DIM)),
            _dev(seq_idx, torch.int32, "seq_idx", (T,)), _dev(pos, torch.int32, "pos", (T,)), T,
            _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
            _dev(seq_lens_after, torch.int32, "seq_lens_after"), _stream(stream))
    return PreparedCall(load().oscar_kv_write, args, (cs, cl, k, v, seq_idx, pos, page_table, seq_lens_after))


def prepare_decode_attn(shape: CacheShape, cache: CacheBuffers, q, page_table, seq_lens, out, workspace,
                        sm_scale: float | None = None, stream=None) -> PreparedCall:
    import torch
    _check_cache(shape, cache)
    B = int(seq_lens.numel())
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    cs, cl = shape.c(), cache.c()
    args = (ctypes.byref(cs), ctypes.byref(cl), _dev(q, torch.bfloat16, "q", (B, shape.num_q_heads, HEAD_DIM)),
            _dev(page_table, torch.int32, "page_table"), int(page_table.shape[1]),
            _dev(seq_lens, torch.int32, "seq_lens", (B,)), B, float(sm_scale),
            _dev(out, torch.bfloat16, "out", (B, shape.num_q_heads, HEAD_DIM)),
            workspace.data_ptr(), workspace.numel(), _stream(stream))
    return PreparedCall(load().oscar_decode_attn, args, (cs, cl, q, page_table, seq_lens, out, workspace))


def prepare_bf16_decode_attn(num_kv_heads: int, num_q_heads: int, pages, q, page_table, seq_lens, out,
                             workspace, sm_scale: float | None = None, stream=None) -> PreparedCall:
    args = _bf16_decode_args(num_kv_heads, num_q_heads, pages, q, page_table, seq_lens, out, workspace,
                             sm_scale, stream)
    return PreparedCall(load().oscar_bf16_decode_attn, args, (pages, q, page_table, seq_lens, out, workspace))


def read_probe_sink_bytes() -> int:
    return int(load().oscar_read_probe_sink_bytes())


def prepare_read_probe(buf, sink, stream=None) -> PreparedCall:
    """oscar_read_probe (measurement aid): one plain read of the whole device
    tensor `buf`; `sink` is a uint8 device tensor of read_probe_sink_bytes()."""
    if not buf.is_cuda or not sink.is_cuda or not buf.is_contiguous():
        raise OscarError("read probe buffers must be contiguous device tensors")
    nbytes = buf.numel() * buf.element_size()
    args = (buf.data_ptr(), nbytes, sink.data_ptr(), sink.numel() * sink.element_size(), _stream(stream))
    return PreparedCall(load().oscar_read_probe, args, (buf, sink))


def prepare_decode_step(shape: CacheShape, cache: CacheBuffers, k, v, seq_idx, pos, seq_lens_after, q, page_table,
                        seq_lens, out, workspace, sm_scale: float | None = None, stream=None) -> PreparedCall:
    args, keep = _decode_step_args(shape, cache, k, v, seq_idx, pos, seq_lens_after, q, page_table, seq_lens,
                                   out, workspace, sm_scale, stream)
    return PreparedCall(load().oscar_decode_step, args, keep)
