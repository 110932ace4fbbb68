"""fp64 oracle for decode attention over bf16 KV caches (one or T query tokens per row).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The GPU library and its Python
binding never import it, and it never imports them.

Two independent formulations live here:
  * ``decode`` -- ctypes wrapper over ``oracle.c``: the plain definition, one query row
    at a time, positions visited in ascending order (see the header of oracle.c for
    the definition and the passages of the pages it follows);
  * ``brute.brute_decode`` -- a dense numpy formulation (full logits matrix over every
    position, explicit -inf mask, np softmax) for tiny shapes.
Both take bf16 tensors as raw uint16 bit patterns in numpy arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

LINEAR = 0
RING = 1

FLAG_QPOS_GE_CTX = 1
FLAG_EVICTED = 2
FLAG_LINEAR_OVER = 4
FLAG_NEGATIVE = 8

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB) or (
            os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P = ctypes.c_void_p
    i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    lib.oracle_decode_f64.argtypes = [ctypes.c_int] * 6 + [P, P, P, P, P, ctypes.c_int, f32, f32,
                                                           P, P, P, ctypes.c_long, P, ctypes.c_int]
    lib.oracle_decode_f64.restype = ctypes.c_int
    lib.oracle_decode_multi_f64.argtypes = [ctypes.c_int] * 7 + [P, P, P, P, P, ctypes.c_int, f32,
                                                                 f32, P, P, P, ctypes.c_long, P,
                                                                 ctypes.c_int]
    lib.oracle_decode_multi_f64.restype = ctypes.c_int
    lib.oracle_append.argtypes = [ctypes.c_int] * 5 + [P, P, P]
    lib.oracle_append.restype = ctypes.c_int
    lib.oracle_valid_positions.argtypes = [i32, i32, i32, i32, i32, P, P]
    lib.oracle_valid_positions.restype = i64
    lib.oracle_row_flags.argtypes = [i32, i32, i32, i32, i32]
    lib.oracle_row_flags.restype = i32
    lib.oracle_split_merge_f64.argtypes = [ctypes.c_long, ctypes.c_int, P, P, ctypes.c_int, P, P]
    lib.oracle_split_merge_f64.restype = f64
    lib.oracle_decode_fp8_multi_f64.argtypes = [ctypes.c_int] * 7 + [P] * 7 + [
        ctypes.c_int, f32, f32, P, P, P, ctypes.c_long, P, ctypes.c_int]
    lib.oracle_decode_fp8_multi_f64.restype = ctypes.c_int
    lib.oracle_append_fp8.argtypes = [ctypes.c_int] * 6 + [P, P, P, P]
    lib.oracle_append_fp8.restype = ctypes.c_int
    lib.oracle_quantize_row_fp8.argtypes = [ctypes.c_int, P, P, P]
    lib.oracle_quantize_row_fp8.restype = None
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f64.restype = f64
    lib.oracle_f32_to_e4m3.argtypes = [f32]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_f64_to_bf16.argtypes = [f64]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_rope_row.argtypes = [ctypes.c_int, P, ctypes.c_long, f64, ctypes.c_int, P, P]
    lib.oracle_rope_row.restype = None
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = f64
    lib.oracle_num_threads_default.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"bf16 inputs are passed as uint16 bit patterns, got {a.dtype}")
    return a


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def num_threads_default() -> int:
    return _load().oracle_num_threads_default()


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits) & 0xFFFF)


def decode(q, k_cache, v_cache, ctx_lens, q_pos, window, softcap, scale, kind, probs_len=0,
           nthreads=0):
    """Plain fp64 decode attention.

    q [B,Hq,D]; k_cache/v_cache [B,Hkv,cap,D] (uint16 bf16 bits; v_cache None: V = K);
    ctx_lens, q_pos [B]; window <= 0: full causal; softcap <= 0 or non-finite: off;
    scale: float32 value.  kind: LINEAR or RING.
    Returns (out [B,Hq,D] f64, lse [B,Hq] f64, probs [B,Hq,probs_len] or None, flags [B]).
    """
    lib = _load()
    q = _u16(q)
    k_cache = _u16(k_cache)
    v_cache = None if v_cache is None else _u16(v_cache)
    B, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_cache.shape
    if Bk != B or Dk != D or (v_cache is not None and v_cache.shape != k_cache.shape):
        raise ValueError("shape mismatch")
    ctx_lens, q_pos = _i32(ctx_lens), _i32(q_pos)
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    probs = np.zeros((B, Hq, probs_len), np.float64) if probs_len > 0 else None
    flags = np.zeros((B,), np.int32)
    rc = lib.oracle_decode_f64(B, Hq, Hkv, D, cap, int(kind), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(ctx_lens), _ptr(q_pos), int(window), float(softcap),
                               float(scale), _ptr(out), _ptr(lse), _ptr(probs), int(probs_len),
                               _ptr(flags), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_decode_f64 failed: {rc}")
    return out, lse, probs, flags


def decode_multi(q, k_cache, v_cache, ctx_lens, q_pos0, window, softcap, scale, kind,
                 probs_len=0, nthreads=0):
    """Plain fp64 decode attention for T consecutive query tokens per batch row.

    q [B,T,Hq,D]; token t of row b sits at position q_pos0[b] + t and is masked at that
    position (causal limit and window of its own), against the same cache rows.
    Returns (out [B,T,Hq,D], lse [B,T,Hq], probs [B,T,Hq,probs_len] or None, flags [B,T]).
    """
    lib = _load()
    q = _u16(q)
    k_cache = _u16(k_cache)
    v_cache = None if v_cache is None else _u16(v_cache)
    B, T, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_cache.shape
    if Bk != B or Dk != D or (v_cache is not None and v_cache.shape != k_cache.shape):
        raise ValueError("shape mismatch")
    ctx_lens, q_pos0 = _i32(ctx_lens), _i32(q_pos0)
    out = np.zeros((B, T, Hq, D), np.float64)
    lse = np.zeros((B, T, Hq), np.float64)
    probs = np.zeros((B, T, Hq, probs_len), np.float64) if probs_len > 0 else None
    flags = np.zeros((B, T), np.int32)
    rc = lib.oracle_decode_multi_f64(B, T, Hq, Hkv, D, cap, int(kind), _ptr(q), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(ctx_lens), _ptr(q_pos0), int(window),
                                     float(softcap), float(scale), _ptr(out), _ptr(lse),
                                     _ptr(probs), int(probs_len), _ptr(flags), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_decode_multi_f64 failed: {rc}")
    return out, lse, probs, flags


def e4m3_to_f64(code: int) -> float:
    """Value of an OCP e4m3 (fn) code (NaN for 0x7f / 0xff)."""
    return _load().oracle_e4m3_to_f64(int(code) & 0xFF)


def f32_to_e4m3(x: float) -> int:
    """Round-to-nearest-even e4m3 code of a float32 value (saturating at +-448)."""
    return int(_load().oracle_f32_to_e4m3(float(np.float32(x))))


def quantize_rows_fp8(x_bits):
    """Quantize bf16 rows (uint16 bits [..., D]) to (codes uint8 [..., D], scales f32 [...])."""
    lib = _load()
    x = _u16(x_bits)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    codes = np.zeros(flat.shape, np.uint8)
    scales = np.zeros((flat.shape[0],), np.float32)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        c = np.zeros((D,), np.uint8)
        sc = np.zeros((1,), np.float32)
        lib.oracle_quantize_row_fp8(D, _ptr(row), _ptr(c), _ptr(sc))
        codes[r] = c
        scales[r] = sc[0]
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1])


def append_fp8(codes, scales, new_rows, pos0, kind):
    """In-place quantizing append of T tokens per row: codes [B,Hkv,cap,D] uint8, scales
    [B,Hkv,cap] float32, new_rows [B,T,Hkv,D] bf16 bits, token t at pos0[b] + t (out-of-range
    positions skipped)."""
    lib = _load()
    for a, dt in ((codes, np.uint8), (scales, np.float32)):
        if not (isinstance(a, np.ndarray) and a.flags.c_contiguous and a.dtype == dt):
            raise TypeError("codes / scales must be C-contiguous uint8 / float32 arrays")
    new_rows = _u16(new_rows)
    B, Hkv, cap, D = codes.shape
    T = new_rows.shape[1]
    if new_rows.shape != (B, T, Hkv, D) or scales.shape != (B, Hkv, cap):
        raise ValueError("shape mismatch")
    rc = lib.oracle_append_fp8(B, T, Hkv, D, cap, int(kind), _ptr(codes), _ptr(scales),
                               _ptr(new_rows), _ptr(_i32(pos0)))
    if rc != 0:
        raise ValueError(f"oracle_append_fp8 failed: {rc}")


def decode_fp8_multi(q, k_codes, k_scales, v_codes, v_scales, ctx_lens, q_pos0, window, softcap,
                     scale, kind, probs_len=0, nthreads=0):
    """decode_multi over fp8 caches (values code * row scale); v_codes None: V = K.
    q [B,T,Hq,D] bf16 bits (a [B,Hq,D] q is taken as T = 1 and returns [B,Hq,D])."""
    lib = _load()
    q = _u16(q)
    single = q.ndim == 3
    if single:
        q = q[:, None]
    B, T, Hq, D = q.shape
    k_codes = np.ascontiguousarray(k_codes, np.uint8)
    k_scales = np.ascontiguousarray(k_scales, np.float32)
    if v_codes is not None:
        v_codes = np.ascontiguousarray(v_codes, np.uint8)
        v_scales = np.ascontiguousarray(v_scales, np.float32)
    Bk, Hkv, cap, Dk = k_codes.shape
    if Bk != B or Dk != D or k_scales.shape != (B, Hkv, cap):
        raise ValueError("shape mismatch")
    ctx_lens, q_pos0 = _i32(ctx_lens), _i32(q_pos0)
    out = np.zeros((B, T, Hq, D), np.float64)
    lse = np.zeros((B, T, Hq), np.float64)
    probs = np.zeros((B, T, Hq, probs_len), np.float64) if probs_len > 0 else None
    flags = np.zeros((B, T), np.int32)
    rc = lib.oracle_decode_fp8_multi_f64(B, T, Hq, Hkv, D, cap, int(kind), _ptr(q), _ptr(k_codes),
                                         _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                                         _ptr(ctx_lens), _ptr(q_pos0), int(window),
                                         float(softcap), float(scale), _ptr(out), _ptr(lse),
                                         _ptr(probs), int(probs_len), _ptr(flags), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_decode_fp8_multi_f64 failed: {rc}")
    if single:
        return out[:, 0], lse[:, 0], None if probs is None else probs[:, 0], flags[:, 0]
    return out, lse, probs, flags


def f64_to_bf16(x: float) -> int:
    """bf16 bits of the double x rounded to nearest, ties to even."""
    return int(_load().oracle_f64_to_bf16(float(x)))


def rope(x_bits, positions, base, rotary_dim):
    """Rotary embedding of bf16 rows x [..., D] (uint16 bits) at positions (broadcast over
    the row index: one position per row of x.reshape(-1, D)).  Returns (bf16 bits, float64
    values before rounding)."""
    lib = _load()
    x = _u16(x_bits)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    pos = np.broadcast_to(np.asarray(positions, np.int64).reshape(-1), (flat.shape[0],))
    out = np.zeros(flat.shape, np.uint16)
    out64 = np.zeros(flat.shape, np.float64)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        o = np.zeros((D,), np.uint16)
        o64 = np.zeros((D,), np.float64)
        lib.oracle_rope_row(D, _ptr(row), int(pos[r]), float(base), int(rotary_dim), _ptr(o),
                            _ptr(o64))
        out[r], out64[r] = o, o64
    return out.reshape(x.shape), out64.reshape(x.shape)


def append_tokens(cache, new_rows, pos0, kind):
    """Append T tokens per row in order t = 0..T-1 at positions pos0[b] + t (a later
    token overwrites an earlier one that lands in the same ring slot)."""
    new_rows = _u16(new_rows)
    B, T = new_rows.shape[:2]
    pos0 = _i32(pos0)
    for t in range(T):
        append(cache, np.ascontiguousarray(new_rows[:, t]), pos0 + t, kind)


def append(cache, new_rows, pos, kind):
    """In-place cache append: cache[b,g,slot(pos_b),:] = new_rows[b,g,:]."""
    lib = _load()
    if not (isinstance(cache, np.ndarray) and cache.flags.c_contiguous and cache.dtype == np.uint16):
        raise TypeError("cache must be a C-contiguous uint16 array (updated in place)")
    new_rows = _u16(new_rows)
    B, Hkv, cap, D = cache.shape
    if new_rows.shape != (B, Hkv, D):
        raise ValueError("new_rows must be [B,Hkv,D]")
    pos = _i32(pos)
    rc = lib.oracle_append(B, Hkv, D, cap, int(kind), _ptr(cache), _ptr(new_rows), _ptr(pos))
    if rc != 0:
        raise ValueError(f"oracle_append failed: {rc}")


def valid_positions(ctx, q_pos, window, kind, cap):
    """(positions, slots) of the valid set of one batch row, ascending."""
    lib = _load()
    n = lib.oracle_valid_positions(int(ctx), int(q_pos), int(window), int(kind), int(cap), None, None)
    pos = np.zeros((max(n, 1),), np.int64)
    slots = np.zeros((max(n, 1),), np.int64)
    lib.oracle_valid_positions(int(ctx), int(q_pos), int(window), int(kind), int(cap), _ptr(pos),
                               _ptr(slots))
    return pos[:n], slots[:n]


def row_flags(ctx, q_pos, window, kind, cap) -> int:
    return int(_load().oracle_row_flags(int(ctx), int(q_pos), int(window), int(kind), int(cap)))


def split_merge(logits, values, starts):
    """fp64 split partials merged by log-sum-exp; returns (out [D], lse)."""
    lib = _load()
    logits = np.ascontiguousarray(logits, np.float64)
    values = np.ascontiguousarray(values, np.float64)
    starts = np.ascontiguousarray(starts, np.int64).astype(np.int64)
    n, D = values.shape
    out = np.zeros((D,), np.float64)
    lse = lib.oracle_split_merge_f64(n, D, _ptr(logits), _ptr(values), len(starts) - 1,
                                     _ptr(starts.astype(np.int64)), _ptr(out))
    return out, lse
