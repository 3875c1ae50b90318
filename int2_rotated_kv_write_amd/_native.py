"""ctypes declarations of the C ABI (include/oscar.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "liboscar_gfx950.so"
_lib = None
NOALLOC_SCRATCH_BYTES = 64 << 20     # OSCAR_NOALLOC_SCRATCH_BYTES of include/oscar.h

c_i32 = ctypes.c_int32
c_ptr = ctypes.c_void_p


class OscarShape(ctypes.Structure):
    _fields_ = [("num_kv_heads", c_i32), ("num_q_heads", c_i32), ("head_dim", c_i32),
                ("page_size", c_i32), ("sink", c_i32), ("recent", c_i32), ("group", c_i32)]


class OscarLayer(ctypes.Structure):
    _fields_ = [("pages", c_ptr), ("k_sink", c_ptr), ("v_sink", c_ptr), ("k_ring", c_ptr),
                ("v_ring", c_ptr), ("u_k", c_ptr), ("u_v", c_ptr),
                ("clip_k", ctypes.c_float), ("clip_v", ctypes.c_float)]


EXPORTS = ("oscar_kv_write", "oscar_decode_workspace_bytes", "oscar_decode_attn", "oscar_decode_step",
           "oscar_decode_attn_noalloc", "oscar_extend_workspace_bytes", "oscar_extend_attn",
           "oscar_cascade_workspace_bytes", "oscar_decode_attn_cascade",
           "oscar_bf16_decode_workspace_bytes", "oscar_bf16_decode_attn",
           "oscar_read_probe_sink_bytes", "oscar_read_probe",
           "oscar_calibrate_layer", "oscar_calibrate_clip", "oscar_status_string", "oscar_last_error")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load() -> ctypes.CDLL:
    """Load the in-tree library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python -m int2_rotated_kv_write_amd.build`")
    lib = ctypes.CDLL(path)
    SP, LP = ctypes.POINTER(OscarShape), ctypes.POINTER(OscarLayer)
    lib.oscar_kv_write.argtypes = [SP, LP, c_ptr, c_ptr, c_ptr, c_ptr, c_i32, c_ptr, c_i32, c_ptr, c_ptr]
    lib.oscar_kv_write.restype = ctypes.c_int
    lib.oscar_decode_workspace_bytes.argtypes = [SP, c_i32, c_i32]
    lib.oscar_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.oscar_decode_attn.argtypes = [SP, LP, c_ptr, c_ptr, c_i32, c_ptr, c_i32, ctypes.c_float,
                                      c_ptr, c_ptr, ctypes.c_size_t, c_ptr]
    lib.oscar_decode_attn.restype = ctypes.c_int
    lib.oscar_decode_attn_noalloc.argtypes = [SP, LP, c_ptr, c_ptr, c_i32, c_ptr, c_i32, ctypes.c_float, c_ptr,
                                              c_ptr]
    lib.oscar_decode_attn_noalloc.restype = ctypes.c_int
    lib.oscar_cascade_workspace_bytes.argtypes = [SP, c_i32, c_i32, c_i32]
    lib.oscar_cascade_workspace_bytes.restype = ctypes.c_size_t
    lib.oscar_decode_attn_cascade.argtypes = [SP, LP, c_ptr, c_ptr, c_i32, c_ptr, c_i32, c_ptr, c_ptr, c_i32, c_i32,
                                              c_i32, ctypes.c_float, c_ptr, c_ptr, ctypes.c_size_t, c_ptr]
    lib.oscar_decode_attn_cascade.restype = ctypes.c_int
    lib.oscar_extend_workspace_bytes.argtypes = [SP, c_i32, c_i32, c_i32]
    lib.oscar_extend_workspace_bytes.restype = ctypes.c_size_t
    lib.oscar_extend_attn.argtypes = [SP, LP, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_i32, c_i32, c_i32, c_ptr, c_i32,
                                      ctypes.c_float, c_ptr, c_ptr, ctypes.c_size_t, c_ptr]
    lib.oscar_extend_attn.restype = ctypes.c_int
    lib.oscar_decode_step.argtypes = [SP, LP, c_ptr, c_ptr, c_ptr, c_ptr, c_i32, c_ptr, c_ptr, c_ptr, c_i32,
                                      c_ptr, c_i32, ctypes.c_float, c_ptr, c_ptr, ctypes.c_size_t, c_ptr]
    lib.oscar_decode_step.restype = ctypes.c_int
    lib.oscar_bf16_decode_workspace_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32]
    lib.oscar_bf16_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.oscar_bf16_decode_attn.argtypes = [c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_i32, c_ptr, c_i32,
                                           ctypes.c_float, c_ptr, c_ptr, ctypes.c_size_t, c_ptr]
    lib.oscar_bf16_decode_attn.restype = ctypes.c_int
    lib.oscar_read_probe_sink_bytes.argtypes = []
    lib.oscar_read_probe_sink_bytes.restype = ctypes.c_size_t
    lib.oscar_read_probe.argtypes = [c_ptr, ctypes.c_size_t, c_ptr, ctypes.c_size_t, c_ptr]
    lib.oscar_read_probe.restype = ctypes.c_int
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oscar_calibrate_layer.argtypes = [c_i32, c_i32, c_i32, dp, dp, dp, ctypes.c_double,
                                          ctypes.c_double, c_ptr, c_ptr,
                                          ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_float), c_i32]
    lib.oscar_calibrate_layer.restype = ctypes.c_int
    lib.oscar_calibrate_clip.argtypes = [c_i32, c_i32, dp, c_ptr, ctypes.c_double, ctypes.POINTER(ctypes.c_float)]
    lib.oscar_calibrate_clip.restype = ctypes.c_int
    lib.oscar_status_string.argtypes = [ctypes.c_int]
    lib.oscar_status_string.restype = ctypes.c_char_p
    lib.oscar_last_error.argtypes = []
    lib.oscar_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib
