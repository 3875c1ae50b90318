"""MI355X (gfx950) OSCAR INT2 KV cache: rotated INT2 KV write and
mixed-precision paged decode attention.

Thin Python binding over the C ABI in include/oscar.h (liboscar_gfx950.so,
built in-tree by ``int2_rotated_kv_write_amd.build``).  PyTorch provides
device memory and streams; every step of the write and decode paths runs in
the library's HIP kernels.  Importing this package does not load the library;
the first call does, and raises if the library is missing.
"""
from ._native import load, library_path
from .api import (
    CacheBuffers, CacheShape, OscarError, allocate_cache, bf16_decode_attn, decode_attn_noalloc, extend_attn,
    extend_workspace_bytes, cascade_workspace_bytes, decode_attn_cascade, prepare_decode_attn_cascade,
    bf16_decode_workspace_bytes, calibrate_clip, calibrate_layer, decode_attn, decode_step, decode_workspace_bytes, kv_write,
    prepare_bf16_decode_attn, prepare_decode_attn, prepare_decode_step, prepare_kv_write, prepare_read_probe,
    read_probe_sink_bytes, status_string,
)

__all__ = [
    "load", "library_path", "CacheShape", "CacheBuffers", "OscarError",
    "allocate_cache", "kv_write", "decode_attn", "decode_workspace_bytes",
    "calibrate_layer", "calibrate_clip", "status_string", "prepare_kv_write", "prepare_decode_attn",
    "bf16_decode_attn", "bf16_decode_workspace_bytes", "prepare_bf16_decode_attn",
    "prepare_read_probe", "read_probe_sink_bytes", "decode_step", "prepare_decode_step",
    "decode_attn_noalloc", "extend_attn", "extend_workspace_bytes",
    "cascade_workspace_bytes", "decode_attn_cascade", "prepare_decode_attn_cascade",
]
