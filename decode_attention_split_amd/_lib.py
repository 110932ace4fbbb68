"""ctypes loader for libgemma_attn.so (the HIP library built from csrc/).

Loading fails loudly: there is no fallback path of any kind.  The library is looked up
next to this file (it is built in-tree by build_lib.py / __graft_entry__.build()).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemma_attn.so")


class ga_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32)]


class ga_decode_opts(ctypes.Structure):
    _fields_ = [("split_keys", ctypes.c_int32), ("impl", ctypes.c_int32),
                ("deterministic", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


# Every symbol include/gemma_attn.h declares.
EXPORTS = ["ga_decode_workspace_bytes", "gemma_attn_decode", "gemma_attn_decode_ex",
           "gemma_attn_decode_append",
           "gemma_kv_append", "gemma_attn_validate", "gemma_attn_debug_ranges",
           "gemma_attn_strerror", "gemma_attn_version",
           "ga_decode_multi_workspace_bytes", "gemma_attn_decode_multi", "gemma_kv_append_multi",
           "gemma_attn_validate_multi", "gemma_kv_append_fp8", "ga_decode_fp8_workspace_bytes",
           "gemma_attn_decode_fp8", "gemma_rope_append", "gemma_attn_decode_rope_append",
           "gemma_rope_table", "gemma_attn_decode_append_fp8", "gemma_attn_decode_noalloc",
           "gemma_stream_read_sink_bytes", "gemma_stream_read"]

_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    SP = ctypes.POINTER(ga_shape)
    OP = ctypes.POINTER(ga_decode_opts)
    lib.ga_decode_workspace_bytes.argtypes = [SP, i32, OP]
    lib.ga_decode_workspace_bytes.restype = sz
    lib.gemma_attn_decode.argtypes = [SP, P, P, P, P, P, i32, f32, f32, P, P, sz, P]
    lib.gemma_attn_decode.restype = i32
    lib.gemma_attn_decode_ex.argtypes = [SP, P, P, P, P, P, i32, f32, f32, P, P, sz, OP, P]
    lib.gemma_attn_decode_ex.restype = i32
    lib.gemma_attn_decode_append.argtypes = [SP, P, P, P, P, P, P, P, P, i32, f32, f32, P, P, sz,
                                             OP, P]
    lib.gemma_attn_decode_append.restype = i32
    lib.gemma_kv_append.argtypes = [SP, P, P, P, P, P, P]
    lib.gemma_kv_append.restype = i32
    lib.gemma_attn_validate.argtypes = [SP, P, P, i32, P, P]
    lib.gemma_attn_validate.restype = i32
    lib.gemma_attn_debug_ranges.argtypes = [SP, P, P, i32, P, P]
    lib.gemma_attn_debug_ranges.restype = i32
    lib.ga_decode_multi_workspace_bytes.argtypes = [SP, i32, i32, OP]
    lib.ga_decode_multi_workspace_bytes.restype = sz
    lib.gemma_attn_decode_multi.argtypes = [SP, i32, P, P, P, P, P, i32, f32, f32, P, P, sz, OP,
                                            P]
    lib.gemma_attn_decode_multi.restype = i32
    lib.gemma_kv_append_multi.argtypes = [SP, i32, P, P, P, P, P, P]
    lib.gemma_kv_append_multi.restype = i32
    lib.gemma_attn_validate_multi.argtypes = [SP, i32, P, P, i32, P, P]
    lib.gemma_attn_validate_multi.restype = i32
    lib.gemma_kv_append_fp8.argtypes = [SP, i32, P, P, P, P, P, P, P, P]
    lib.gemma_kv_append_fp8.restype = i32
    lib.ga_decode_fp8_workspace_bytes.argtypes = [SP, i32, i32, OP]
    lib.ga_decode_fp8_workspace_bytes.restype = sz
    lib.gemma_attn_decode_fp8.argtypes = [SP, i32, P, P, P, P, P, P, P, i32, f32, f32, P, P, sz,
                                          OP, P]
    lib.gemma_attn_decode_fp8.restype = i32
    lib.gemma_rope_append.argtypes = [SP, i32, P, P, P, P, P, P, P, f32, i32, P]
    lib.gemma_rope_append.restype = i32
    lib.gemma_attn_decode_rope_append.argtypes = [SP, P, P, P, P, P, P, P, P, P, i32, f32, f32,
                                                  P, i32, P, P, sz, OP, P]
    lib.gemma_attn_decode_rope_append.restype = i32
    lib.gemma_rope_table.argtypes = [i32, P, f32, i32, i32, P, P]
    lib.gemma_rope_table.restype = i32
    lib.gemma_attn_decode_append_fp8.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, i32, f32, f32,
                                                 P, P, sz, OP, P]
    lib.gemma_attn_decode_append_fp8.restype = i32
    lib.gemma_attn_decode_noalloc.argtypes = [SP, P, P, P, P, P, i32, f32, f32, P, OP, P]
    lib.gemma_attn_decode_noalloc.restype = i32
    lib.gemma_stream_read_sink_bytes.argtypes = []
    lib.gemma_stream_read_sink_bytes.restype = sz
    lib.gemma_stream_read.argtypes = [P, sz, P, P]
    lib.gemma_stream_read.restype = i32
    lib.gemma_attn_strerror.argtypes = [i32]
    lib.gemma_attn_strerror.restype = ctypes.c_char_p
    lib.gemma_attn_version.argtypes = []
    lib.gemma_attn_version.restype = i32
    _lib = lib
    return lib
