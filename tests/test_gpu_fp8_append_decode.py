"""GPU: the quantizing append fused with single-token decode over fp8 caches.

gemma_attn_decode_append_fp8 promises the bits of gemma_kv_append_fp8 (one token) then
gemma_attn_decode_fp8: the same codes and scales in the caches and the same output.  On
the vector kernel and on the global matrix-core kernel one launch does both (each
work-group quantizes the new rows with the append's arithmetic and substitutes them for the
appended key).  Each case runs both routes on copies of the same caches and compares
bit for bit; one case also checks the caches and the output against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_split_amd import api, synth

from common import assert_parity, default_scale, log
from test_gpu_fp8 import FP8_NAN, Fp8Inputs

pytestmark = pytest.mark.gpu


def _new_rows(seed, B, Hkv, D, k_eq_v):
    gen = synth.generator(seed)
    kn = synth.normal_bf16(gen, (B, Hkv, D)) * 3
    kn[1, 0] = 0  # an all-zero row: codes 0, scale 0
    vn = None if k_eq_v else synth.normal_bf16(gen, (B, Hkv, D))
    return kn, vn


def _poison_appended(inp, ctx, cap, kind):
    """NaN codes and scales in the slots the call appends to: the two calls overwrite them
    before reading, the one call must never use what it loads from them."""
    for b, c in enumerate(ctx):
        if c > 0 and (kind == api.RING or c - 1 < cap):
            slot = (c - 1) % cap if kind == api.RING else c - 1
            for codes, scales in ((inp.kc_d, inp.ks_d), (inp.vc_d, inp.vs_d)):
                if codes is not None:
                    codes[b, :, slot] = FP8_NAN
                    scales[b, :, slot] = float("nan")


def _both_routes(inp, kn, vn, window, softcap, kind, max_ctx, split_keys=0, impl=api.IMPL_AUTO,
                 q_pos=None):
    q = inp.q[:, 0].contiguous()
    pos = inp.ctx_t - 1
    q_pos = pos if q_pos is None else q_pos
    c = lambda t: None if t is None else t.clone()
    kd, vd = kn.cuda(), None if vn is None else vn.cuda()
    scale = default_scale(kn.shape[-1])
    # one call
    f = [c(inp.kc_d), c(inp.ks_d), c(inp.vc_d), c(inp.vs_d)]
    out_f = api.decode_append_fp8(q, f[0], f[1], f[2], f[3], kd, vd, pos, inp.ctx_t, q_pos, window,
                                  softcap, scale, kind, max_ctx=max_ctx, split_keys=split_keys,
                                  deterministic=True, impl=impl)
    # the two calls
    r = [c(inp.kc_d), c(inp.ks_d), c(inp.vc_d), c(inp.vs_d)]
    api.kv_append_fp8(r[0], r[1], r[2], r[3], kd[:, None], None if vd is None else vd[:, None],
                      pos, kind)
    out_r = api.decode_fp8(q, r[0], r[1], r[2], r[3], inp.ctx_t, q_pos, window, softcap, scale,
                           kind, max_ctx=max_ctx, split_keys=split_keys, deterministic=True,
                           impl=impl)
    torch.cuda.synchronize()
    for a, b, what in zip(f, r, ("K codes", "K scales", "V codes", "V scales")):
        if a is not None:
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what
    assert torch.equal(out_f.view(torch.int32), out_r.view(torch.int32)), "output bits"
    return out_f, f


@pytest.mark.parametrize("D,G,Hkv,k_eq_v,kind,impl", [
    (256, 2, 4, False, api.RING, api.IMPL_AUTO),     # 12B sliding geometry
    (128, 4, 2, False, api.LINEAR, api.IMPL_AUTO),
    (256, 1, 2, True, api.RING, api.IMPL_AUTO),      # K = V on the vector kernel
    (256, 8, 1, False, api.RING, api.IMPL_AUTO),
    (512, 16, 1, True, api.LINEAR, api.IMPL_AUTO),   # global geometry: matrix cores
    (512, 16, 1, True, api.LINEAR, api.IMPL_VALU),   # global geometry on the vector kernel
])
@pytest.mark.parametrize("split_keys", [0, 64])
def test_fused_fp8_append_decode_equals_two_calls(D, G, Hkv, k_eq_v, kind, impl, split_keys):
    if kind == api.RING:
        cap = window = 100
        ctx = [0, 1, 37, 100, 503]   # an empty row (nothing appended), partial, full, wrapped
        max_ctx = max(ctx)
    else:
        cap, window = 300, 0
        ctx = [0, 1, 150, 299, 300]
        max_ctx = cap
    log(f"fp8 append+decode D={D} G={G} Hkv={Hkv} K=V={k_eq_v} kind={kind} impl={impl} "
        f"split={split_keys}")
    inp = Fp8Inputs(D + G + kind + split_keys, len(ctx), 1, G * Hkv, Hkv, D, cap, k_eq_v,
                    ctx).to_device()
    _poison_appended(inp, ctx, cap, kind)
    kn, vn = _new_rows(D + G, len(ctx), Hkv, D, k_eq_v)
    _both_routes(inp, kn, vn, window, 30.0 if G % 2 == 0 else 0.0, kind, max_ctx, split_keys,
                 impl)


def test_fused_fp8_global_stale_slot_and_rows_without_keys():
    """The global geometry on the matrix cores: the appended slots hold NaN codes and scales
    before the call (the two calls overwrite them before reading; the one call must take
    the new row's codes and scale instead of what it loads from the slot), a row with
    q_pos = -1 appends without attending (no work-group of its own: work-group u appends),
    an empty row appends nothing; balanced over the chip and with split sizes 64 and 512."""
    D, G, Hkv, cap = 512, 16, 1, 2048
    ctx = [0, 5, 1, 700, 2048, 1500]
    inp = Fp8Inputs(4242, len(ctx), 1, G * Hkv, Hkv, D, cap, True, ctx).to_device()
    _poison_appended(inp, ctx, cap, api.LINEAR)
    kn, _ = _new_rows(4243, len(ctx), Hkv, D, True)
    q_pos = inp.ctx_t - 1
    q_pos[1] = -1
    for split in (0, 64, 512):
        log(f"fp8 global fused append: split={split}")
        out, _ = _both_routes(inp, kn, None, 0, 0.0, api.LINEAR, cap, split,
                              api.IMPL_MFMA if split else api.IMPL_AUTO, q_pos=q_pos)
        assert torch.isfinite(out).all()


def test_fused_fp8_global_more_units_than_one_launch():
    """1100 rows of one KV head: two matrix-core launches, the quantizing append fused
    into both (the appended slots NaN-poisoned before the call)."""
    D, G, Hkv, cap, B = 512, 16, 1, 64, 1100
    ctx = synth.uniform_int(synth.generator(4244), B, 1, cap).numpy().astype(np.int32).tolist()
    inp = Fp8Inputs(4245, B, 1, G * Hkv, Hkv, D, cap, True, ctx).to_device()
    _poison_appended(inp, ctx, cap, api.LINEAR)
    kn, _ = _new_rows(4246, B, Hkv, D, True)
    log("fp8 global fused append: B=1100")
    _both_routes(inp, kn, None, 0, 0.0, api.LINEAR, cap)


def test_fused_fp8_global_layer_full_size_sampled_rows():
    """The 12B fp8 global layer at full size in the launch the bench times (quantizing
    append + decode in one matrix-core launch): the new slot's codes and scale and the
    output of sampled rows against the oracle."""
    from decode_attention_split_amd import workloads as wl
    w = wl.FP8_GLOBAL
    g = w.layers[0]
    B, D, C = w.batch, g.head_dim, g.capacity
    ctx = synth.uniform_int(synth.generator(w.seed), B, w.ctx_lo, w.ctx_hi).numpy() \
        .astype(np.int32)
    gd = synth.generator(92, device="cuda")
    kc = torch.full((B, 1, C, D), FP8_NAN, dtype=torch.uint8, device="cuda")
    ks = torch.full((B, 1, C), float("nan"), dtype=torch.float32, device="cuda")
    ctx_t = torch.from_numpy(ctx).cuda()
    chunk = 1024
    for p0 in range(0, int(ctx.max()) - 1, chunk):
        kn = synth.normal_bf16(gd, (B, chunk, 1, D), device="cuda")
        # rows past ctx - 2 land beyond each row's old context: their slots are rewritten
        # below or never read
        api.kv_append_fp8(kc, ks, None, None, kn, None,
                          torch.full((B,), p0, dtype=torch.int32, device="cuda"), g.kind)
    # the slots the call appends to hold NaN codes and scales until then
    rows_d = torch.arange(B, device="cuda")
    kc[rows_d, 0, ctx_t.long() - 1] = FP8_NAN
    ks[rows_d, 0, ctx_t.long() - 1] = float("nan")
    kn = synth.normal_bf16(gd, (B, 1, D), device="cuda")
    q = synth.normal_bf16(gd, (B, g.num_q_heads, D), device="cuda")
    out = api.decode_append_fp8(q, kc, ks, None, None, kn, None, ctx_t - 1, ctx_t, ctx_t - 1,
                                g.window, g.softcap, g.q_scale, g.kind, max_ctx=C)
    torch.cuda.synchronize()
    rows = sorted({0, int(np.argmax(ctx)), int(np.argmin(ctx))})
    log(f"fused fp8 global rows {rows} ctx {ctx[rows].tolist()}")
    kcr, ksr = kc[rows].cpu().numpy(), ks[rows].cpu().numpy()
    for i, b in enumerate(rows):
        c, s = oracle.quantize_rows_fp8(synth.bits(kn[b].cpu()))
        slot = int(ctx[b]) - 1
        assert np.array_equal(kcr[i, :, slot], c) and np.array_equal(ksr[i, :, slot], s)
    ref, _, _, _ = oracle.decode_fp8_multi(synth.bits(q[rows].cpu())[:, None], kcr, ksr, None,
                                           None, ctx[rows], ctx[rows] - 1, g.window, g.softcap,
                                           g.q_scale, g.kind)
    assert_parity(out[rows].unsqueeze(1), ref, "fused fp8 global full size")


def test_fused_fp8_append_decode_matches_oracle():
    """Caches after the one call equal the oracle's quantizing append, and the output the
    oracle's decode over those caches."""
    D, G, Hkv, W = 256, 2, 4, 100
    ctx = [2, 100, 503]
    inp = Fp8Inputs(77, len(ctx), 1, G * Hkv, Hkv, D, W, False, ctx).to_device()
    kn, vn = _new_rows(78, len(ctx), Hkv, D, False)
    out, f = _both_routes(inp, kn, vn, W, 0.0, api.RING, max(ctx), split_keys=64)
    pos = np.asarray(ctx, np.int32) - 1
    oracle.append_fp8(inp.kc, inp.ks, synth.bits(kn)[:, None], pos, api.RING)
    oracle.append_fp8(inp.vc, inp.vs, synth.bits(vn)[:, None], pos, api.RING)
    assert np.array_equal(f[0].cpu().numpy(), inp.kc)
    assert np.array_equal(f[1].cpu().numpy().view(np.uint32), inp.ks.view(np.uint32))
    assert np.array_equal(f[2].cpu().numpy(), inp.vc)
    assert np.array_equal(f[3].cpu().numpy().view(np.uint32), inp.vs.view(np.uint32))
    ref, _ = inp.oracle(W, 0.0, default_scale(D), api.RING)
    assert_parity(out.unsqueeze(1), ref, "fused fp8 append + decode")


def test_fused_fp8_sliding_layer_full_size_sampled_rows():
    """The 12B fp8 sliding layer at full size in the launch the bench times: the cache filled
    by a quantizing append of the previous 1023 tokens, then the current token appended and
    attended in one call; sampled rows against the oracle (the new slot's codes and scales,
    and the output over the resulting cache)."""
    from decode_attention_split_amd import workloads as wl
    w = wl.G4_12B_SLIDING
    g = w.layers[0]
    B, Hkv, D, W = w.batch, g.num_kv_heads, g.head_dim, g.capacity
    ctx = synth.uniform_int(synth.generator(w.seed), B, w.ctx_lo, w.ctx_hi).numpy() \
        .astype(np.int32)
    gd = synth.generator(91, device="cuda")
    kc = torch.empty((B, Hkv, W, D), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    ks = torch.empty((B, Hkv, W), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    ctx_t = torch.from_numpy(ctx).cuda()
    old = synth.normal_bf16(gd, (B, W - 1, Hkv, D), device="cuda")
    api.kv_append_fp8(kc, ks, vc, vs, old, synth.normal_bf16(gd, old.shape, device="cuda"),
                      ctx_t - W, api.RING)
    kn = synth.normal_bf16(gd, (B, Hkv, D), device="cuda")
    vn = synth.normal_bf16(gd, (B, Hkv, D), device="cuda")
    q = synth.normal_bf16(gd, (B, g.num_q_heads, D), device="cuda")
    out = api.decode_append_fp8(q, kc, ks, vc, vs, kn, vn, ctx_t - 1, ctx_t, ctx_t - 1,
                                g.window, g.softcap, g.q_scale, g.kind, max_ctx=w.ctx_hi)
    torch.cuda.synchronize()
    rows = sorted({0, 1, int(np.argmax(ctx)), int(np.argmin(ctx))})
    log(f"fused fp8 sliding rows {rows}")
    kcr, ksr = kc[rows].cpu().numpy(), ks[rows].cpu().numpy()
    vcr, vsr = vc[rows].cpu().numpy(), vs[rows].cpu().numpy()
    for i, b in enumerate(rows):
        slot = (int(ctx[b]) - 1) % W
        c, s = oracle.quantize_rows_fp8(synth.bits(kn[b].cpu()))
        assert np.array_equal(kcr[i, :, slot], c) and np.array_equal(ksr[i, :, slot], s)
        c, s = oracle.quantize_rows_fp8(synth.bits(vn[b].cpu()))
        assert np.array_equal(vcr[i, :, slot], c) and np.array_equal(vsr[i, :, slot], s)
    ref, _, _, _ = oracle.decode_fp8_multi(synth.bits(q[rows].cpu())[:, None], kcr, ksr, vcr, vsr,
                                           ctx[rows], ctx[rows] - 1, g.window, g.softcap,
                                           g.q_scale, g.kind)
    assert_parity(out[rows].unsqueeze(1), ref, "fused fp8 sliding full size")
