"""C-ABI boundary checks that need no GPU.

The library must load and export every function include/gemma_attn.h declares, and
every host-side argument check must fire before any HIP call (so these calls never
touch device memory: the pointers passed are never dereferenced).
"""
import ctypes
import math
import os
import re

import pytest

from decode_attention_split_amd import _lib
from decode_attention_split_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemma_attn.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert "gemma_attn_decode" in names and "gemma_kv_append" in names
    assert sorted(names) == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    lib = _lib.load()
    assert lib.gemma_attn_version() >= 100
    for code in [0] + list(api.ERRORS) + [-999, 5]:
        s = lib.gemma_attn_strerror(code)
        assert s is not None and len(s) > 0


def shape(B=2, Hq=16, Hkv=8, D=256, cap=1024, kind=api.RING, max_ctx=0):
    return api.make_shape(B, Hq, Hkv, D, cap, kind, max_ctx)


def call_decode(s, window=1024, softcap=0.0, scale=0.0625, v=FAKE, ws=FAKE, ws_bytes=1 << 40,
                q=FAKE, k=FAKE, ctx=FAKE, qpos=FAKE, out=FAKE, opts=None):
    lib = _lib.load()
    P = ctypes.c_void_p
    return lib.gemma_attn_decode_ex(ctypes.byref(s), P(q), P(k), P(v) if v else None, P(ctx),
                                    P(qpos), window, softcap, scale, P(out), P(ws) if ws else None,
                                    ws_bytes, ctypes.byref(opts) if opts else None, None)


def no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.parametrize("kw,code", [
    (dict(s=shape(D=64)), -3),
    (dict(s=shape(D=384)), -3),
    (dict(s=shape(D=384)), -3),
    (dict(s=shape(Hq=12, Hkv=8)), -4),
    (dict(s=shape(Hq=24, Hkv=1)), -4),    # G = 24 is not supported
    (dict(s=shape(Hq=6, Hkv=2)), -4),     # G = 3 is not supported
    (dict(s=shape(B=-1)), -2),
    (dict(s=shape(Hkv=0)), -2),
    (dict(s=shape(cap=0)), -2),
    (dict(s=shape(kind=2)), -5),
    (dict(s=shape(cap=512), window=1024), -6),             # ring window > W
    (dict(s=shape(cap=512, max_ctx=4096), window=0), -6),  # full attention, ctx may exceed W
    (dict(s=shape(kind=api.LINEAR, cap=512, max_ctx=513), window=0), -13),
    (dict(s=shape(max_ctx=-5)), -13),
    (dict(s=shape(), scale=math.inf), -8),
    (dict(s=shape(), scale=math.nan), -8),
    (dict(s=shape(), q=0), -1),
    (dict(s=shape(), k=0), -1),
    (dict(s=shape(), ctx=0), -1),
    (dict(s=shape(), qpos=0), -1),
    (dict(s=shape(), out=0), -1),
    (dict(s=shape(), q=FAKE + 8), -1),                     # not 16-byte aligned
    (dict(s=shape(B=2), ws=0, ws_bytes=0), -7),        # 16 units x 8 splits need partials
    (dict(s=shape(B=2), ws_bytes=16), -7),
    (dict(s=shape(), opts=api.make_opts(split_keys=100)), -12),
    (dict(s=shape(), opts=api.make_opts(split_keys=32)), -12),
    (dict(s=shape(), opts=api.make_opts(impl=7)), -12),
    (dict(s=shape(), opts=api.make_opts(impl=api.IMPL_MFMA)), -12),  # MFMA: D512 G16 only
])
def test_decode_rejects_bad_arguments_before_any_launch(kw, code):
    assert call_decode(**kw) == code


def test_reserved_option_fields_must_be_zero():
    o = api.make_opts()
    o.reserved[3] = 1
    assert call_decode(shape(), opts=o) == -12


def test_deterministic_option_is_a_flag():
    o = api.make_opts(deterministic=True)
    assert o.deterministic == 1
    o.deterministic = 2
    assert call_decode(shape(), opts=o) == -12


@pytest.mark.skipif(not no_gpu(), reason="checks the no-device path")
def test_valid_decode_without_a_gpu_reports_arch_error():
    assert call_decode(shape()) == -10
    s = shape(B=0)
    assert call_decode(s, ws=0, ws_bytes=0) == -10


def test_workspace_bytes_closed_form():
    lib = _lib.load()
    # B 64, Hq 16, D 256, ring W = w = 1024, split 256 keys -> S = 4 splits
    s = shape(B=64, Hq=16, Hkv=8, D=256, cap=1024, max_ctx=8192)
    o = api.make_opts(split_keys=256)
    n = lib.ga_decode_workspace_bytes(ctypes.byref(s), 1024, ctypes.byref(o))
    assert n == 64 * 16 * 4 * (256 + 2) * 4
    # one split covers every row: no workspace
    o = api.make_opts(split_keys=1024)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s), 1024, ctypes.byref(o)) == 0
    # a window shorter than the ring bounds the keys: w = 100 -> one 128-key split
    o = api.make_opts(split_keys=128)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s), 100, ctypes.byref(o)) == 0
    # linear C 32768, full causal, split 512 on the vector kernel: S = 64
    s = shape(B=16, Hq=16, Hkv=1, D=512, cap=32768, kind=api.LINEAR)
    o = api.make_opts(split_keys=512, impl=api.IMPL_VALU)
    valu512 = 16 * 16 * 64 * 514 * 4
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s), 0, ctypes.byref(o)) == valu512
    # K = V global geometry: AUTO may pick the matrix-core path, whose workspace is one
    # partial slot per work-group (16 heads x (512 + 2) floats) plus B * Hkv + 1 ints of
    # prefix sums.  Balanced: with B * Hkv <= 3/4 of the 256 CUs the grid is 256 work-
    # groups, one per CU; the query covers the larger of the two kernels
    mfma = 256 * 16 * 514 * 4 + 17 * 4
    o = api.make_opts(impl=api.IMPL_MFMA)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s), 0, ctypes.byref(o)) == mfma
    auto = lib.ga_decode_workspace_bytes(ctypes.byref(s), 0, None)
    valu = lib.ga_decode_workspace_bytes(ctypes.byref(s), 0,
                                         ctypes.byref(api.make_opts(impl=api.IMPL_VALU)))
    assert auto == max(mfma, valu)
    # past 3/4 of the CUs in units the grid is 256 + B * Hkv work-groups
    s2 = shape(B=200, Hq=16, Hkv=1, D=512, cap=4096, kind=api.LINEAR)
    o = api.make_opts(impl=api.IMPL_MFMA)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s2), 0, ctypes.byref(o)) == \
        (256 + 200) * 16 * 514 * 4 + 201 * 4
    # a split size keeps the matrix cores: every unit at most ceil(C / split) work-groups,
    # one partial each; AUTO sizes for either kernel
    o = api.make_opts(split_keys=512)
    mfma512 = 16 * 64 * 16 * 514 * 4 + 17 * 4
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s), 0, ctypes.byref(o)) == \
        max(mfma512, valu512)
    o = api.make_opts(split_keys=512, impl=api.IMPL_MFMA)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s), 0, ctypes.byref(o)) == mfma512
    # more units than one launch takes (1024): launches of 1024 / Hkv rows reuse one
    # workspace sized for a launch
    s3 = shape(B=3000, Hq=16, Hkv=1, D=512, cap=2048, kind=api.LINEAR)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s3), 0, ctypes.byref(o)) == \
        1024 * 4 * 16 * 514 * 4 + 1025 * 4
    # invalid shape -> SIZE_MAX
    bad = shape(D=100)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(bad), 0, None) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("kw,code", [
    (dict(v_cache=FAKE, v_new=0), -9),
    (dict(v_cache=0, v_new=FAKE), -9),
    (dict(k_cache=0), -1),
    (dict(pos=0), -1),
    (dict(D=100), -3),
    (dict(kind=5), -5),
    (dict(Hkv=0), -2),
])
def test_append_rejects_bad_arguments(kw, code):
    lib = _lib.load()
    args = dict(k_cache=FAKE, v_cache=FAKE, k_new=FAKE, v_new=FAKE, pos=FAKE, D=256, kind=api.RING,
                Hkv=8)
    args.update(kw)
    s = api.make_shape(4, 8, args["Hkv"], args["D"], 1024, args["kind"])
    P = ctypes.c_void_p
    rc = lib.gemma_kv_append(ctypes.byref(s), P(args["k_cache"]) if args["k_cache"] else None,
                             P(args["v_cache"]) if args["v_cache"] else None, P(args["k_new"]),
                             P(args["v_new"]) if args["v_new"] else None,
                             P(args["pos"]) if args["pos"] else None, None)
    assert rc == code


def test_append_and_debug_calls_without_a_gpu():
    if not no_gpu():
        pytest.skip("checks the no-device path")
    lib = _lib.load()
    s = api.make_shape(4, 8, 8, 256, 1024, api.RING)
    P = ctypes.c_void_p
    assert lib.gemma_kv_append(ctypes.byref(s), P(FAKE), None, P(FAKE), None, P(FAKE), None) == -10
    assert lib.gemma_attn_validate(ctypes.byref(s), P(FAKE), P(FAKE), 1024, P(FAKE), None) == -10
    assert lib.gemma_attn_debug_ranges(ctypes.byref(s), P(FAKE), P(FAKE), 1024, P(FAKE),
                                       None) == -10


# ------------------------------------------------------------------ multi-token entry points

def call_decode_multi(s, T, window=1024, ws=FAKE, ws_bytes=1 << 40, opts=None, v=FAKE):
    lib = _lib.load()
    P = ctypes.c_void_p
    return lib.gemma_attn_decode_multi(ctypes.byref(s), T, P(FAKE), P(FAKE), P(v) if v else None,
                                       P(FAKE), P(FAKE), window, 0.0, 0.0625, P(FAKE),
                                       P(ws) if ws else None, ws_bytes,
                                       ctypes.byref(opts) if opts else None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(s=shape(), T=0), -2),                                   # no tokens
    (dict(s=shape(), T=5000), -14),                               # beyond the token limit
    # ring of W = w = 1024 that the context can overrun: 8 tokens need 1031 slots
    (dict(s=shape(cap=1024, max_ctx=8192), T=8), -6),
    (dict(s=shape(cap=1031, max_ctx=8192), T=8, ws=0, ws_bytes=0), -7),
    # matrix cores for several tokens: head_dim 512 only with K = V
    (dict(s=shape(D=512, Hq=16, Hkv=1, cap=4096, kind=api.LINEAR), T=8, v=FAKE + 4096,
          opts=api.make_opts(impl=api.IMPL_MFMA)), -12),
    (dict(s=shape(cap=1031, max_ctx=8192), T=8, opts=api.make_opts(split_keys=100)), -12),
])
def test_decode_multi_rejects_bad_arguments_before_any_launch(kw, code):
    assert call_decode_multi(**kw) == code


@pytest.mark.skipif(not no_gpu(), reason="checks the no-device path")
def test_valid_decode_multi_without_a_gpu_reports_arch_error():
    # a ring of exactly w slots is fine while the context cannot exceed it
    assert call_decode_multi(shape(cap=1024, max_ctx=1024), 8) == -10
    assert call_decode_multi(shape(cap=1031, max_ctx=8192), 8) == -10


def test_multi_workspace_closed_form():
    """B 4, 16q/8kv (G = 2), hd256, ring 1031 for w 1024, T = 8 tokens.
    Vector kernel: 4 tokens per unit (2 heads x 4 tokens = 8 rows), 2 chunks; a unit's keys
    are at most w + 4 - 1 = 1027; 64 units want 4 splits of ceil(1027 / 4) = 257 -> 320
    keys, S = ceil(1027 / 320) = 4.  Matrix cores: 8 tokens per unit (16 rows), 1 chunk,
    at most w + 8 - 1 = 1031 keys; 32 units want 2048 / 4 = 512 four-wave splits, 16 each,
    of ceil(1031 / 16) = 65 -> 80 keys (whole 16-key tiles), S = ceil(1031 / 80) = 13.
    Partials: B * T * Hq * S * (D + 2) floats; the automatic choice sizes for the
    larger."""
    lib = _lib.load()
    s = shape(B=4, cap=1031, max_ctx=8192)
    valu = api.make_opts(impl=api.IMPL_VALU)
    mfma = api.make_opts(impl=api.IMPL_MFMA)
    n_v = lib.ga_decode_multi_workspace_bytes(ctypes.byref(s), 8, 1024, ctypes.byref(valu))
    n_m = lib.ga_decode_multi_workspace_bytes(ctypes.byref(s), 8, 1024, ctypes.byref(mfma))
    assert n_v == 4 * 8 * 16 * 4 * (256 + 2) * 4
    assert n_m == 4 * 8 * 16 * 13 * (256 + 2) * 4
    assert lib.ga_decode_multi_workspace_bytes(ctypes.byref(s), 8, 1024, None) == max(n_v, n_m)
    # T = 1 is the single-token plan
    o = api.make_opts()
    assert lib.ga_decode_multi_workspace_bytes(ctypes.byref(s), 1, 1024, ctypes.byref(o)) == \
        lib.ga_decode_workspace_bytes(ctypes.byref(s), 1024, ctypes.byref(o))


def test_append_multi_argument_checks():
    lib = _lib.load()
    P = ctypes.c_void_p
    s = shape()
    assert lib.gemma_kv_append_multi(ctypes.byref(s), 0, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                     P(FAKE), None) == -2
    assert lib.gemma_kv_append_multi(ctypes.byref(s), 4, P(FAKE), None, P(FAKE), P(FAKE),
                                     P(FAKE), None) == -9
    assert lib.gemma_attn_validate_multi(ctypes.byref(shape(cap=1024, max_ctx=8192)), 8, P(FAKE),
                                         P(FAKE), 1024, P(FAKE), None) == -6


def test_rope_table_argument_checks():
    lib = _lib.load()
    P = ctypes.c_void_p
    assert lib.gemma_rope_table(-1, P(FAKE), 1e4, 256, 256, P(FAKE), None) == -2  # batch < 0
    assert lib.gemma_rope_table(4, P(FAKE), 1e4, 255, 256, P(FAKE), None) == -2   # R odd
    assert lib.gemma_rope_table(4, P(FAKE), 1e4, -2, 256, P(FAKE), None) == -2    # R < 0
    assert lib.gemma_rope_table(4, P(FAKE), 1e4, 258, 256, P(FAKE), None) == -2   # R > D
    assert lib.gemma_rope_table(4, P(FAKE), 1e4, 128, 100, P(FAKE), None) == -3   # D
    assert lib.gemma_rope_table(4, P(FAKE), 1e4, 128, 1024, P(FAKE), None) == -3
    assert lib.gemma_rope_table(4, P(FAKE), 0.0, 256, 256, P(FAKE), None) == -12  # base <= 0
    assert lib.gemma_rope_table(4, P(FAKE), math.inf, 256, 256, P(FAKE), None) == -12
    assert lib.gemma_rope_table(4, None, 1e4, 256, 256, P(FAKE), None) == -1
    assert lib.gemma_rope_table(4, P(FAKE), 1e4, 256, 256, None, None) == -1
    assert lib.gemma_rope_table(4, P(FAKE), 1e4, 256, 256, P(FAKE + 8), None) == -1  # align
    # nothing to compute: OK without touching a device
    assert lib.gemma_rope_table(0, None, 1e4, 256, 256, None, None) == 0
    assert lib.gemma_rope_table(4, None, 1e4, 0, 256, None, None) == 0


def test_decode_rope_append_argument_checks():
    lib = _lib.load()
    P = ctypes.c_void_p
    s = shape()

    def call(q_out=FAKE, k_new=FAKE, table=FAKE, R=256, v=FAKE, v_new=FAKE):
        return lib.gemma_attn_decode_rope_append(
            ctypes.byref(s), P(FAKE), P(q_out) if q_out else None, P(FAKE),
            P(v) if v else None, P(k_new) if k_new else None, P(v_new) if v_new else None,
            P(FAKE), P(FAKE), P(FAKE), 1024, 0.0, 0.0625, P(table) if table else None, R, P(FAKE),
            P(FAKE), 1 << 40, None, None)
    assert call(q_out=0) == -1
    assert call(q_out=FAKE + 8) == -1
    assert call(k_new=0) == -1
    assert call(R=255) == -12
    assert call(R=258) == -12      # > head_dim
    assert call(R=-2) == -12
    assert call(table=0) == -1     # a rotary part needs the table
    assert call(table=FAKE + 8) == -1
    assert call(v_new=0) == -9     # v_cache without v_new
    if no_gpu():
        assert call(table=0, R=0) == -10  # valid: reaches the device check
        assert call() == -10


def test_decode_append_fp8_argument_checks():
    lib = _lib.load()
    P = ctypes.c_void_p
    s = shape()

    def call(k_new=FAKE, v_codes=FAKE, v_scales=FAKE, v_new=FAKE, pos=FAKE):
        return lib.gemma_attn_decode_append_fp8(
            ctypes.byref(s), P(FAKE), P(FAKE), P(FAKE), P(v_codes) if v_codes else None,
            P(v_scales) if v_scales else None, P(k_new) if k_new else None,
            P(v_new) if v_new else None, P(pos) if pos else None, P(FAKE), P(FAKE), 1024, 0.0,
            0.0625, P(FAKE), P(FAKE), 1 << 40, None, None)
    assert call(k_new=0) == -1
    assert call(pos=0) == -1
    assert call(v_new=0) == -9              # V codes without V rows
    assert call(v_scales=0) == -9           # V codes without V scales
    if no_gpu():
        assert call() == -10
        assert call(v_codes=0, v_scales=0, v_new=0) == -10  # K = V


def test_noalloc_refuses_a_call_beyond_its_scratch_before_any_launch():
    """gemma_attn_decode_noalloc returns GA_ERR_SCRATCH (nothing launched, no device call)
    when the plan's workspace exceeds its fixed scratch, and the host checks of
    gemma_attn_decode_ex before that."""
    lib = _lib.load()
    P = ctypes.c_void_p
    s = shape(B=4, Hq=16, Hkv=1, D=512, cap=1 << 16, kind=api.LINEAR)
    o = api.make_opts(split_keys=64, impl=api.IMPL_MFMA)
    assert lib.ga_decode_workspace_bytes(ctypes.byref(s), 0, ctypes.byref(o)) > \
        api.NOALLOC_SCRATCH_BYTES
    rc = lib.gemma_attn_decode_noalloc(ctypes.byref(s), P(FAKE), P(FAKE), None, P(FAKE), P(FAKE),
                                       0, 0.0, 1.0, P(FAKE), ctypes.byref(o), None)
    assert rc == -15
    bad = shape(D=100)
    assert lib.gemma_attn_decode_noalloc(ctypes.byref(bad), P(FAKE), P(FAKE), None, P(FAKE),
                                         P(FAKE), 0, 0.0, 1.0, P(FAKE), None, None) == -3
    assert lib.gemma_attn_decode_noalloc(ctypes.byref(shape()), None, P(FAKE), None, P(FAKE),
                                         P(FAKE), 1024, 0.0, 1.0, P(FAKE), None, None) == -1
