"""Python binding of libgemma_attn: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/gemma_attn.h).  torch provides device memory and the current stream; this
module checks tensor dtypes, devices and contiguity, passes raw pointers, and raises
GemmaAttnError when the library returns a non-zero status.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

LINEAR = 0
RING = 1
IMPL_AUTO, IMPL_VALU, IMPL_MFMA = 0, 1, 2

GA_OK = 0
ERRORS = {
    -1: "GA_ERR_NULL", -2: "GA_ERR_DIMS", -3: "GA_ERR_HEAD_DIM", -4: "GA_ERR_GQA",
    -5: "GA_ERR_KIND", -6: "GA_ERR_WINDOW", -7: "GA_ERR_WORKSPACE", -8: "GA_ERR_SCALE",
    -9: "GA_ERR_V_MISMATCH", -10: "GA_ERR_ARCH", -11: "GA_ERR_LAUNCH", -12: "GA_ERR_OPTS",
    -13: "GA_ERR_MAX_CTX", -14: "GA_ERR_TOO_LARGE", -15: "GA_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 32 << 20  # GA_NOALLOC_SCRATCH_BYTES
FLAG_QPOS_GE_CTX, FLAG_EVICTED, FLAG_LINEAR_OVER, FLAG_NEGATIVE, FLAG_OVER_MAX_CTX = 1, 2, 4, 8, 16


class GemmaAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        msg = _lib.load().gemma_attn_strerror(self.code).decode()
        super().__init__(f"{where}: {ERRORS.get(self.code, self.code)} ({msg})")


def _check(code: int, where: str):
    if code != GA_OK:
        raise GemmaAttnError(code, where)


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, capacity, kind, max_ctx=0):
    return _lib.ga_shape(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim),
                         int(capacity), int(kind), int(max_ctx))


def make_opts(split_keys=0, impl=IMPL_AUTO, deterministic=False):
    o = _lib.ga_decode_opts()
    o.split_keys = int(split_keys)
    o.impl = int(impl)
    o.deterministic = int(bool(deterministic))
    return o


def _ptr(t: Optional[torch.Tensor]):
    # the prototypes declare c_void_p: a plain int converts without building an object
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream=None):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:  # the current stream's handle without a Stream object
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype, ndim=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def version() -> int:
    return int(_lib.load().gemma_attn_version())


def workspace_bytes(shape, window: int, split_keys: int = 0, impl: int = IMPL_AUTO) -> int:
    lib = _lib.load()
    opts = make_opts(split_keys, impl)
    n = lib.ga_decode_workspace_bytes(ctypes.byref(shape), int(window), ctypes.byref(opts))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid shape/window/options for gemma_attn_decode")
    return int(n)


def workspace_bytes_multi(shape, num_tokens: int, window: int, split_keys: int = 0) -> int:
    lib = _lib.load()
    opts = make_opts(split_keys)
    n = lib.ga_decode_multi_workspace_bytes(ctypes.byref(shape), int(num_tokens), int(window),
                                            ctypes.byref(opts))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid shape/tokens/window/options for gemma_attn_decode_multi")
    return int(n)


def shape_of(q, k_cache, kind, max_ctx=0):
    B, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k_cache {tuple(k_cache.shape)} disagree")
    return make_shape(B, Hq, Hkv, D, cap, kind, max_ctx)


def _decode_common(q, k_cache, v_cache, ctx_lens, q_pos, window, kind, out, workspace, max_ctx,
                   split_keys, impl, deterministic, need_workspace=True):
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    if v_cache is not None:
        _need(v_cache, "v_cache", torch.bfloat16, 4)
        if v_cache.shape != k_cache.shape:
            raise ValueError("v_cache must have the shape of k_cache")
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    shape = shape_of(q, k_cache, kind, max_ctx)
    if ctx_lens.numel() != shape.batch or q_pos.numel() != shape.batch:
        raise ValueError("ctx_lens and q_pos must have one entry per batch row")
    if out is None:
        out = torch.empty((shape.batch, shape.num_q_heads, shape.head_dim), dtype=torch.float32,
                          device=q.device)
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (shape.batch, shape.num_q_heads, shape.head_dim):
            raise ValueError("out must be [B, Hq, D]")
    opts = make_opts(split_keys, impl, deterministic)
    if not need_workspace:
        return shape, out, opts, None
    if workspace is None:  # a given workspace is checked against its size by the library
        lib = _lib.load()
        need = lib.ga_decode_workspace_bytes(ctypes.byref(shape), int(window),
                                             ctypes.byref(opts))
        if need == ctypes.c_size_t(-1).value:
            need = 0  # let the library report the precise error
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    return shape, out, opts, workspace


def decode(q, k_cache, v_cache, ctx_lens, q_pos, window: int, softcap: float, scale: float,
           kind: int, out=None, workspace=None, max_ctx: int = 0, split_keys: int = 0,
           impl: int = IMPL_AUTO, deterministic: bool = False, stream=None):
    """Single-token decode attention; returns out [B, Hq, D] float32 (see gemma_attn.h).

    v_cache None means K = V (k_cache serves as keys and values).  workspace, when
    given, is a uint8 device tensor of at least workspace_bytes(...) bytes; otherwise
    one is allocated here with torch (the library itself never allocates).
    """
    shape, out, opts, workspace = _decode_common(q, k_cache, v_cache, ctx_lens, q_pos, window,
                                                 kind, out, workspace, max_ctx, split_keys, impl,
                                                 deterministic)
    ws_bytes = 0 if workspace is None else workspace.numel()
    rc = _lib.load().gemma_attn_decode_ex(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_lens), _ptr(q_pos),
        int(window), float(softcap), float(scale), _ptr(out), _ptr(workspace), ws_bytes,
        ctypes.byref(opts), _stream_handle(stream))
    _check(rc, "gemma_attn_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, ctx_lens, q_pos, window: int, softcap: float,
                   scale: float, kind: int, out=None, max_ctx: int = 0, split_keys: int = 0,
                   impl: int = IMPL_AUTO, deterministic: bool = False, stream=None):
    """decode() without a workspace: gemma_attn_decode_noalloc uses the library's fixed
    device scratch (see gemma_attn.h); nothing is allocated here except `out` when it is
    not given."""
    shape, out, opts, _ = _decode_common(q, k_cache, v_cache, ctx_lens, q_pos, window, kind,
                                         out, None, max_ctx, split_keys, impl, deterministic,
                                         need_workspace=False)
    rc = _lib.load().gemma_attn_decode_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_lens), _ptr(q_pos),
        int(window), float(softcap), float(scale), _ptr(out), ctypes.byref(opts),
        _stream_handle(stream))
    _check(rc, "gemma_attn_decode_noalloc")
    return out


def decode_append(q, k_cache, v_cache, k_new, v_new, pos, ctx_lens, q_pos, window: int,
                  softcap: float, scale: float, kind: int, out=None, workspace=None,
                  max_ctx: int = 0, split_keys: int = 0, impl: int = IMPL_AUTO,
                  deterministic: bool = False, stream=None):
    """kv_append(k_cache, v_cache, k_new, v_new, pos) then decode(...), in one launch."""
    shape, out, opts, workspace = _decode_common(q, k_cache, v_cache, ctx_lens, q_pos, window,
                                                 kind, out, workspace, max_ctx, split_keys, impl,
                                                 deterministic)
    _need(k_new, "k_new", torch.bfloat16, 3)
    if (v_cache is None) != (v_new is None):
        _check(-9, "gemma_attn_decode_append")
    if v_new is not None:
        _need(v_new, "v_new", torch.bfloat16, 3)
    _need(pos, "pos", torch.int32, 1)
    B, Hkv, _, D = k_cache.shape
    if tuple(k_new.shape) != (B, Hkv, D) or (v_new is not None and v_new.shape != k_new.shape) \
            or pos.numel() != B:
        raise ValueError("k_new / v_new must be [B, Hkv, D] and pos [B]")
    ws_bytes = 0 if workspace is None else workspace.numel()
    rc = _lib.load().gemma_attn_decode_append(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        _ptr(pos), _ptr(ctx_lens), _ptr(q_pos), int(window), float(softcap), float(scale),
        _ptr(out), _ptr(workspace), ws_bytes, ctypes.byref(opts), _stream_handle(stream))
    _check(rc, "gemma_attn_decode_append")
    return out


def rope_table(pos, rope_base: float, rotary_dim: int, head_dim: int, out=None, stream=None):
    """cos / sin of every turning rotate-half pair of a head_dim head at pos[b]: float64
    [B, rotary_dim / 2, 2] (see gemma_rope_table)."""
    _need(pos, "pos", torch.int32, 1)
    B = pos.numel()
    if out is None:
        out = torch.empty((B, max(rotary_dim, 0) // 2, 2), dtype=torch.float64,
                          device=pos.device)
    elif out.dtype != torch.float64 or not out.is_contiguous() or \
            tuple(out.shape) != (B, rotary_dim // 2, 2):
        raise ValueError("out must be a contiguous float64 [B, rotary_dim / 2, 2] tensor")
    rc = _lib.load().gemma_rope_table(int(B), _ptr(pos), float(rope_base), int(rotary_dim),
                                      int(head_dim), _ptr(out), _stream_handle(stream))
    _check(rc, "gemma_rope_table")
    return out


def decode_rope_append(q, q_out, k_cache, v_cache, k_new, v_new, pos, ctx_lens, q_pos,
                       window: int, softcap: float, scale: float, kind: int, table,
                       rotary_dim: int, out=None, workspace=None, max_ctx: int = 0,
                       split_keys: int = 0, impl: int = IMPL_AUTO, deterministic: bool = False,
                       stream=None):
    """rope_append(q, q_out, ...) of one token then decode(q_out, ...), one launch where the
    vector kernel serves the shape; table = rope_table(pos, base, rotary_dim, D) (see
    gemma_attn_decode_rope_append)."""
    if table is not None and (table.dtype != torch.float64 or not table.is_contiguous() or
                              tuple(table.shape) != (pos.numel(), rotary_dim // 2, 2)):
        raise ValueError("table must be rope_table(pos, base, rotary_dim, head_dim)")
    shape, out, opts, workspace = _decode_common(q, k_cache, v_cache, ctx_lens, q_pos, window,
                                                 kind, out, workspace, max_ctx, split_keys, impl,
                                                 deterministic)
    _need(q_out, "q_out", torch.bfloat16, 3)
    if q_out.shape != q.shape:
        raise ValueError("q_out must have q's shape")
    _need(k_new, "k_new", torch.bfloat16, 3)
    if (v_cache is None) != (v_new is None):
        _check(-9, "gemma_attn_decode_rope_append")
    if v_new is not None:
        _need(v_new, "v_new", torch.bfloat16, 3)
    _need(pos, "pos", torch.int32, 1)
    B, Hkv, _, D = k_cache.shape
    if tuple(k_new.shape) != (B, Hkv, D) or (v_new is not None and v_new.shape != k_new.shape) \
            or pos.numel() != B:
        raise ValueError("k_new / v_new must be [B, Hkv, D] and pos [B]")
    ws_bytes = 0 if workspace is None else workspace.numel()
    rc = _lib.load().gemma_attn_decode_rope_append(
        ctypes.byref(shape), _ptr(q), _ptr(q_out), _ptr(k_cache), _ptr(v_cache), _ptr(k_new),
        _ptr(v_new), _ptr(pos), _ptr(ctx_lens), _ptr(q_pos), int(window), float(softcap),
        float(scale), _ptr(table), int(rotary_dim), _ptr(out), _ptr(workspace), ws_bytes,
        ctypes.byref(opts), _stream_handle(stream))
    _check(rc, "gemma_attn_decode_rope_append")
    return out


def decode_multi(q, k_cache, v_cache, ctx_lens, q_pos, window: int, softcap: float, scale: float,
                 kind: int, out=None, workspace=None, max_ctx: int = 0, split_keys: int = 0,
                 deterministic: bool = False, impl: int = IMPL_AUTO, stream=None):
    """T query tokens per row: q [B, T, Hq, D], token t at position q_pos[b] + t; returns
    out [B, T, Hq, D] float32 (see gemma_attn_decode_multi in gemma_attn.h)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    if v_cache is not None:
        _need(v_cache, "v_cache", torch.bfloat16, 4)
        if v_cache.shape != k_cache.shape:
            raise ValueError("v_cache must have the shape of k_cache")
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    B, T, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k_cache {tuple(k_cache.shape)} disagree")
    if ctx_lens.numel() != B or q_pos.numel() != B:
        raise ValueError("ctx_lens and q_pos must have one entry per batch row")
    shape = make_shape(B, Hq, Hkv, D, cap, kind, max_ctx)
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    else:
        _need(out, "out", torch.float32, 4)
        if tuple(out.shape) != (B, T, Hq, D):
            raise ValueError("out must be [B, T, Hq, D]")
    opts = make_opts(split_keys, impl, deterministic)
    lib = _lib.load()
    if workspace is None:  # a given workspace is checked against its size by the library
        need = lib.ga_decode_multi_workspace_bytes(ctypes.byref(shape), int(T), int(window),
                                                   ctypes.byref(opts))
        if need == ctypes.c_size_t(-1).value:
            need = 0  # let the library report the precise error
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    ws_bytes = 0 if workspace is None else workspace.numel()
    rc = lib.gemma_attn_decode_multi(
        ctypes.byref(shape), int(T), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_lens),
        _ptr(q_pos), int(window), float(softcap), float(scale), _ptr(out), _ptr(workspace),
        ws_bytes, ctypes.byref(opts), _stream_handle(stream))
    _check(rc, "gemma_attn_decode_multi")
    return out


def kv_append_multi(k_cache, v_cache, k_new, v_new, pos, kind: int, stream=None):
    """T tokens per row: k_new / v_new [B, T, Hkv, D] at positions pos[b] + t, in order."""
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(k_new, "k_new", torch.bfloat16, 4)
    if (v_cache is None) != (v_new is None):
        _check(-9, "gemma_kv_append_multi")
    if v_cache is not None:
        _need(v_cache, "v_cache", torch.bfloat16, 4)
        _need(v_new, "v_new", torch.bfloat16, 4)
        if v_cache.shape != k_cache.shape or v_new.shape != k_new.shape:
            raise ValueError("V tensors must have the shapes of the K tensors")
    _need(pos, "pos", torch.int32, 1)
    B, Hkv, cap, D = k_cache.shape
    T = k_new.shape[1]
    if tuple(k_new.shape) != (B, T, Hkv, D) or pos.numel() != B:
        raise ValueError("k_new must be [B, T, Hkv, D] and pos [B]")
    shape = make_shape(B, Hkv, Hkv, D, cap, kind)
    rc = _lib.load().gemma_kv_append_multi(ctypes.byref(shape), int(T), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(pos),
                                           _stream_handle(stream))
    _check(rc, "gemma_kv_append_multi")


def validate_multi(shape, num_tokens: int, ctx_lens, q_pos, window: int, stream=None):
    """Per-token precondition flags (FLAG_*) as an int32 device tensor [B, T]."""
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    flags = torch.empty((shape.batch, int(num_tokens)), dtype=torch.int32,
                        device=ctx_lens.device)
    rc = _lib.load().gemma_attn_validate_multi(ctypes.byref(shape), int(num_tokens),
                                               _ptr(ctx_lens), _ptr(q_pos), int(window),
                                               _ptr(flags), _stream_handle(stream))
    _check(rc, "gemma_attn_validate_multi")
    return flags


def workspace_bytes_fp8(shape, num_tokens: int, window: int, split_keys: int = 0) -> int:
    lib = _lib.load()
    opts = make_opts(split_keys)
    n = lib.ga_decode_fp8_workspace_bytes(ctypes.byref(shape), int(num_tokens), int(window),
                                          ctypes.byref(opts))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid shape/tokens/window/options for gemma_attn_decode_fp8")
    return int(n)


def kv_append_fp8(k_codes, k_scales, v_codes, v_scales, k_new, v_new, pos, kind: int,
                  stream=None):
    """Quantizing append: k_new / v_new bf16 [B, T, Hkv, D] (or [B, Hkv, D] for T = 1) into
    uint8 codes [B, Hkv, cap, D] and float32 scales [B, Hkv, cap] at positions pos[b] + t."""
    _need(k_codes, "k_codes", torch.uint8, 4)
    _need(k_scales, "k_scales", torch.float32, 3)
    if k_new.dim() == 3:
        k_new = k_new.unsqueeze(1)
        v_new = None if v_new is None else v_new.unsqueeze(1)
    _need(k_new, "k_new", torch.bfloat16, 4)
    if (v_codes is None) != (v_new is None) or (v_codes is None) != (v_scales is None):
        _check(-9, "gemma_kv_append_fp8")
    if v_codes is not None:
        _need(v_codes, "v_codes", torch.uint8, 4)
        _need(v_scales, "v_scales", torch.float32, 3)
        _need(v_new, "v_new", torch.bfloat16, 4)
        if v_codes.shape != k_codes.shape or v_new.shape != k_new.shape:
            raise ValueError("V tensors must have the shapes of the K tensors")
    _need(pos, "pos", torch.int32, 1)
    B, Hkv, cap, D = k_codes.shape
    T = k_new.shape[1]
    if tuple(k_new.shape) != (B, T, Hkv, D) or tuple(k_scales.shape) != (B, Hkv, cap) \
            or pos.numel() != B:
        raise ValueError("k_new must be [B, T, Hkv, D], k_scales [B, Hkv, cap] and pos [B]")
    shape = make_shape(B, Hkv, Hkv, D, cap, kind)
    rc = _lib.load().gemma_kv_append_fp8(ctypes.byref(shape), int(T), _ptr(k_codes),
                                         _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                                         _ptr(k_new), _ptr(v_new), _ptr(pos),
                                         _stream_handle(stream))
    _check(rc, "gemma_kv_append_fp8")


def decode_fp8(q, k_codes, k_scales, v_codes, v_scales, ctx_lens, q_pos, window: int,
               softcap: float, scale: float, kind: int, out=None, workspace=None,
               max_ctx: int = 0, split_keys: int = 0, deterministic: bool = False,
               impl: int = IMPL_AUTO, stream=None):
    """Decode over fp8 caches; q [B, Hq, D] (one token) or [B, T, Hq, D] (T tokens at
    q_pos[b] + t); returns out of the same shape, float32 (see gemma_attn_decode_fp8)."""
    single = q.dim() == 3
    q4 = q.unsqueeze(1) if single else q
    _need(q4, "q", torch.bfloat16, 4)
    _need(k_codes, "k_codes", torch.uint8, 4)
    _need(k_scales, "k_scales", torch.float32, 3)
    if v_codes is not None:
        _need(v_codes, "v_codes", torch.uint8, 4)
        _need(v_scales, "v_scales", torch.float32, 3)
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    B, T, Hq, D = q4.shape
    Bk, Hkv, cap, Dk = k_codes.shape
    if Bk != B or Dk != D or tuple(k_scales.shape) != (B, Hkv, cap):
        raise ValueError("q, k_codes and k_scales disagree")
    if ctx_lens.numel() != B or q_pos.numel() != B:
        raise ValueError("ctx_lens and q_pos must have one entry per batch row")
    shape = make_shape(B, Hq, Hkv, D, cap, kind, max_ctx)
    want = (B, Hq, D) if single else (B, T, Hq, D)
    if out is None:
        out = torch.empty(want, dtype=torch.float32, device=q.device)
    else:
        _need(out, "out", torch.float32, len(want))
        if tuple(out.shape) != want:
            raise ValueError(f"out must be {list(want)}")
    opts = make_opts(split_keys, impl, deterministic)
    lib = _lib.load()
    if workspace is None:  # a given workspace is checked against its size by the library
        need = lib.ga_decode_fp8_workspace_bytes(ctypes.byref(shape), int(T), int(window),
                                                 ctypes.byref(opts))
        if need == ctypes.c_size_t(-1).value:
            need = 0  # let the library report the precise error
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    ws_bytes = 0 if workspace is None else workspace.numel()
    rc = lib.gemma_attn_decode_fp8(
        ctypes.byref(shape), int(T), _ptr(q4), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
        _ptr(v_scales), _ptr(ctx_lens), _ptr(q_pos), int(window), float(softcap), float(scale),
        _ptr(out), _ptr(workspace), ws_bytes, ctypes.byref(opts), _stream_handle(stream))
    _check(rc, "gemma_attn_decode_fp8")
    return out


def decode_append_fp8(q, k_codes, k_scales, v_codes, v_scales, k_new, v_new, pos, ctx_lens,
                      q_pos, window: int, softcap: float, scale: float, kind: int, out=None,
                      workspace=None, max_ctx: int = 0, split_keys: int = 0,
                      deterministic: bool = False, impl: int = IMPL_AUTO, stream=None):
    """kv_append_fp8 of one token then decode_fp8 of one token, in one launch where the
    vector kernel serves the shape (see gemma_attn_decode_append_fp8); q [B, Hq, D]."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_codes, "k_codes", torch.uint8, 4)
    _need(k_scales, "k_scales", torch.float32, 3)
    _need(k_new, "k_new", torch.bfloat16, 3)
    if (v_codes is None) != (v_new is None) or (v_codes is None) != (v_scales is None):
        _check(-9, "gemma_attn_decode_append_fp8")
    if v_codes is not None:
        _need(v_codes, "v_codes", torch.uint8, 4)
        _need(v_scales, "v_scales", torch.float32, 3)
        _need(v_new, "v_new", torch.bfloat16, 3)
        if v_codes.shape != k_codes.shape or v_scales.shape != k_scales.shape or \
                v_new.shape != k_new.shape:
            raise ValueError("V tensors must have the shapes of the K tensors")
    _need(pos, "pos", torch.int32, 1)
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    B, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_codes.shape
    if Bk != B or Dk != D or tuple(k_scales.shape) != (B, Hkv, cap) or \
            tuple(k_new.shape) != (B, Hkv, D):
        raise ValueError("q, k_codes, k_scales and k_new disagree")
    if ctx_lens.numel() != B or q_pos.numel() != B or pos.numel() != B:
        raise ValueError("ctx_lens, q_pos and pos must have one entry per batch row")
    shape = make_shape(B, Hq, Hkv, D, cap, kind, max_ctx)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (B, Hq, D):
            raise ValueError("out must be [B, Hq, D]")
    opts = make_opts(split_keys, impl, deterministic)
    lib = _lib.load()
    if workspace is None:  # a given workspace is checked against its size by the library
        need = lib.ga_decode_fp8_workspace_bytes(ctypes.byref(shape), 1, int(window),
                                                 ctypes.byref(opts))
        if need == ctypes.c_size_t(-1).value:
            need = 0  # let the library report the precise error
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    ws_bytes = 0 if workspace is None else workspace.numel()
    rc = lib.gemma_attn_decode_append_fp8(
        ctypes.byref(shape), _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
        _ptr(v_scales), _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(ctx_lens), _ptr(q_pos),
        int(window), float(softcap), float(scale), _ptr(out), _ptr(workspace), ws_bytes,
        ctypes.byref(opts), _stream_handle(stream))
    _check(rc, "gemma_attn_decode_append_fp8")
    return out


def rope_append(q, q_out, k_cache, v_cache, k_new, v_new, pos, kind: int, rope_base: float,
                rotary_dim: int, stream=None):
    """Rotary embedding of q (-> q_out, may be q) and k_new fused with the append of T
    tokens per row at pos[b] + t; q [B, Hq, D] or [B, T, Hq, D], k_new / v_new [B, Hkv, D]
    or [B, T, Hkv, D] (see gemma_rope_append)."""
    single = q.dim() == 3
    q4 = q.unsqueeze(1) if single else q
    o4 = q_out.unsqueeze(1) if single else q_out
    kn = None if k_new is None else (k_new.unsqueeze(1) if k_new.dim() == 3 else k_new)
    vn = None if v_new is None else (v_new.unsqueeze(1) if v_new.dim() == 3 else v_new)
    _need(q4, "q", torch.bfloat16, 4)
    _need(o4, "q_out", torch.bfloat16, 4)
    _need(pos, "pos", torch.int32, 1)
    B, T, Hq, D = q4.shape
    if (v_cache is None) != (vn is None):
        _check(-9, "gemma_rope_append")
    if k_cache is None:  # rotate q only
        if kn is not None or v_cache is not None:
            raise ValueError("k_new / v_cache need a k_cache")
        Hkv, cap = Hq, 1
    else:
        _need(k_cache, "k_cache", torch.bfloat16, 4)
        _need(kn, "k_new", torch.bfloat16, 4)
        if v_cache is not None:
            _need(v_cache, "v_cache", torch.bfloat16, 4)
            _need(vn, "v_new", torch.bfloat16, 4)
        Bk, Hkv, cap, Dk = k_cache.shape
        if tuple(kn.shape) != (B, T, Hkv, D) or Bk != B or Dk != D or \
                (vn is not None and (vn.shape != kn.shape or v_cache.shape != k_cache.shape)):
            raise ValueError("shape mismatch (new rows [B,T,Hkv,D], caches [B,Hkv,cap,D])")
    if o4.shape != q4.shape or pos.numel() != B:
        raise ValueError("q_out must have q's shape and pos one entry per row")
    shape = make_shape(B, Hq, Hkv, D, cap, kind)
    rc = _lib.load().gemma_rope_append(ctypes.byref(shape), int(T), _ptr(q4), _ptr(o4),
                                       _ptr(k_cache), _ptr(v_cache), _ptr(kn), _ptr(vn),
                                       _ptr(pos), float(rope_base), int(rotary_dim),
                                       _stream_handle(stream))
    _check(rc, "gemma_rope_append")
    return q_out


def kv_append(k_cache, v_cache, k_new, v_new, pos, kind: int, stream=None):
    """cache[b, g, slot(pos_b), :] <- new[b, g, :] for K (and V unless K = V)."""
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(k_new, "k_new", torch.bfloat16, 3)
    if (v_cache is None) != (v_new is None):
        _check(-9, "gemma_kv_append")
    if v_cache is not None:
        _need(v_cache, "v_cache", torch.bfloat16, 4)
        _need(v_new, "v_new", torch.bfloat16, 3)
        if v_cache.shape != k_cache.shape or v_new.shape != k_new.shape:
            raise ValueError("V tensors must have the shapes of the K tensors")
    _need(pos, "pos", torch.int32, 1)
    B, Hkv, cap, D = k_cache.shape
    if tuple(k_new.shape) != (B, Hkv, D) or pos.numel() != B:
        raise ValueError("k_new must be [B, Hkv, D] and pos [B]")
    shape = make_shape(B, Hkv, Hkv, D, cap, kind)
    rc = _lib.load().gemma_kv_append(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_new), _ptr(v_new), _ptr(pos), _stream_handle(stream))
    _check(rc, "gemma_kv_append")


def validate(shape, ctx_lens, q_pos, window: int, flags=None, stream=None):
    """Per-row precondition flags (FLAG_*) as an int32 device tensor."""
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    if flags is None:
        flags = torch.empty((shape.batch,), dtype=torch.int32, device=ctx_lens.device)
    rc = _lib.load().gemma_attn_validate(ctypes.byref(shape), _ptr(ctx_lens), _ptr(q_pos),
                                         int(window), _ptr(flags), _stream_handle(stream))
    _check(rc, "gemma_attn_validate")
    return flags


def debug_ranges(shape, ctx_lens, q_pos, window: int, stream=None):
    """(lo, hi, slot(lo), n) per row, as the decode kernels compute them: int32 [B, 4]."""
    _need(ctx_lens, "ctx_lens", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    out = torch.empty((shape.batch, 4), dtype=torch.int32, device=ctx_lens.device)
    rc = _lib.load().gemma_attn_debug_ranges(ctypes.byref(shape), _ptr(ctx_lens), _ptr(q_pos),
                                             int(window), _ptr(out), _stream_handle(stream))
    _check(rc, "gemma_attn_debug_ranges")
    return out


def stream_read(src, sink=None, stream=None):
    """One streaming read of the whole uint8/any-dtype device tensor `src` (its byte size a
    multiple of 1024) with gemma_stream_read; returns the sink tensor."""
    lib = _lib.load()
    if sink is None:
        sink = torch.empty((lib.gemma_stream_read_sink_bytes(),), dtype=torch.uint8,
                           device=src.device)
    nbytes = src.numel() * src.element_size()
    _check(lib.gemma_stream_read(_ptr(src), nbytes, _ptr(sink), _stream_handle(stream)),
           "gemma_stream_read")
    return sink
