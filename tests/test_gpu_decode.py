"""GPU: decode attention against the fp64 oracle, and the invariants of the method.

Every parity case poisons the slots outside each row's valid set with bf16 NaN, so a
stray read shows up as a NaN output.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_split_amd import api, synth
from decode_attention_split_amd import workloads as wl

from common import (LayerInputs, assert_parity, default_scale, errors, f32, gen_layer, log,
                    oracle_out, poison_invalid_slots)

pytestmark = pytest.mark.gpu


def run(inp, window, softcap, scale, kind, **kw):
    out = api.decode(inp.q, inp.k, inp.v, inp.ctx_t, inp.qpos_t, window, softcap, scale, kind,
                     **kw)
    torch.cuda.synchronize()
    return out


def layer_case(seed, B, geom: wl.LayerGeom, ctx_lo, ctx_hi, ctx=None, poison=True):
    inp = gen_layer(seed, B, geom.num_q_heads, geom.num_kv_heads, geom.head_dim, geom.capacity,
                    geom.k_eq_v, ctx_lo, ctx_hi, ctx)
    if poison:
        poison_invalid_slots(inp, geom.window, geom.kind, geom.capacity)
    return inp.to_device()


# ------------------------------------------------------------------ the five workloads

def test_tiny_sliding_decode():
    w = wl.TINY
    g = w.layers[0]
    inp = layer_case(w.seed, w.batch, g, w.ctx_lo, w.ctx_hi)
    log(f"tiny: {w.name}")
    out = run(inp, g.window, g.softcap, g.q_scale, g.kind)
    assert_parity(out, oracle_out(inp, g.window, g.softcap, g.q_scale, g.kind), "tiny")


@pytest.mark.parametrize("w", [wl.G3_1B_SLIDING, wl.G4_12B_SLIDING, wl.HD128_SLIDING],
                         ids=["g3_1b", "g4_12b", "hd128"])
def test_sliding_layer_full_size(w):
    g = w.layers[0]
    log(f"full size: {w.name}")
    inp = layer_case(w.seed, w.batch, g, w.ctx_lo, w.ctx_hi)
    out = run(inp, g.window, g.softcap, g.q_scale, g.kind)
    assert_parity(out, oracle_out(inp, g.window, g.softcap, g.q_scale, g.kind), w.name)


def test_global_layer_full_size_sampled_rows():
    w = wl.G4_12B_GLOBAL
    g = w.layers[0]
    log(f"full size: {w.name}")
    inp = layer_case(w.seed, w.batch, g, w.ctx_lo, w.ctx_hi)  # never-valid slots NaN
    out = run(inp, g.window, g.softcap, g.q_scale, g.kind)
    assert torch.isfinite(out).all(), "a never-valid slot was read"
    rows = sorted({0, 1, int(np.argmax(inp.ctx)), int(np.argmin(inp.ctx))})
    ref = oracle_out(inp, g.window, g.softcap, g.q_scale, g.kind, rows=rows)
    assert_parity(out[rows], ref, f"{w.name} rows {rows}")


def test_global_layer_at_128k_context():
    """The K = V global geometry at a 128K-token linear cache (128 MiB of keys per row):
    a full row and a ragged one, 16 query heads each, never-valid slots NaN-poisoned, the
    whole output against the oracle; balanced over the chip and in splits of 4096 keys."""
    g = wl.global_geom(16, 131072)
    inp = layer_case(8128, 2, g, 1, 131072, ctx=[131072, 70001])
    log("global layer, 128K context")
    ref = oracle_out(inp, g.window, g.softcap, g.q_scale, g.kind)
    for split in (0, 4096):
        out = run(inp, g.window, g.softcap, g.q_scale, g.kind, split_keys=split,
                  impl=api.IMPL_MFMA)
        assert torch.isfinite(out).all(), "a never-valid slot was read"
        assert_parity(out, ref, f"global 128K split={split}")


@pytest.mark.parametrize("layer", [0, 5, 46, 47])
def test_hybrid_step_layer_sampled_rows(layer):
    w = wl.HYBRID_48
    g = w.layers[layer]
    log(f"hybrid layer {layer}: {'global' if g.k_eq_v else 'sliding'}")
    inp = layer_case(wl.layer_seed(w, layer), w.batch, g, w.ctx_lo, w.ctx_hi)  # NaN-poisoned
    out = run(inp, g.window, g.softcap, g.q_scale, g.kind, max_ctx=min(w.ctx_hi, g.capacity)
              if g.kind == api.LINEAR else w.ctx_hi)
    assert torch.isfinite(out).all(), "a never-valid slot was read"
    rows = sorted({0, 7, int(np.argmax(inp.ctx)), int(np.argmin(inp.ctx))})
    ref = oracle_out(inp, g.window, g.softcap, g.q_scale, g.kind, rows=rows)
    assert_parity(out[rows], ref, f"hybrid layer {layer} rows {rows}")


# ------------------------------------------------------------------ geometry sweep

@pytest.mark.parametrize("D", [128, 256, 512])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("k_eq_v", [False, True])
def test_geometry_sweep(D, G, k_eq_v):
    """Small shapes that still span several splits and steps with ragged tails."""
    Hkv = 2 if G <= 4 else 1
    B = 3
    kind = api.RING if not k_eq_v else api.LINEAR
    cap = 200 if kind == api.RING else 700
    window = 150 if kind == api.RING else 0
    geom = wl.LayerGeom(G * Hkv, Hkv, D, kind, cap, window, k_eq_v, 30.0 if G % 2 == 0 else 0.0)
    seed = D * 100 + G * 10 + int(k_eq_v)
    inp = layer_case(seed, B, geom, 1, 3 * cap if kind == api.RING else cap, ctx=None)
    log(f"sweep D={D} G={G} k_eq_v={k_eq_v} ctx={inp.ctx.tolist()}")
    ref = oracle_out(inp, window, geom.softcap, geom.q_scale, kind)
    for split in [0, 64, 128]:
        out = run(inp, window, geom.softcap, geom.q_scale, kind, split_keys=split,
                  max_ctx=int(inp.ctx.max()) if kind == api.RING else cap)
        assert_parity(out, ref, f"split={split}")


# ------------------------------------------------------------------ cross-layer cache sharing

def test_shared_layers_attend_over_the_owner_cache():
    """A 12-layer stack whose last 4 layers share caches: one fused step appends once per
    owner, and each layer's output equals the oracle over its owner's cache after the
    step (a sharing layer sees the token its owner appended)."""
    from decode_attention_split_amd.hybrid import HybridKVCache
    layers = wl.hybrid_layers(12, wl.sliding_geom(8, 4, 128), wl.global_geom(16, 1024))
    src = wl.kv_share_sources(layers, 4)
    B = 3
    ctx = np.array([1, 300, 1024], np.int32)
    gd = synth.generator(96)
    fill = lambda li, name, shape: synth.normal_bf16(gd, shape).cuda()
    cache = HybridKVCache(layers, B, 1024, device="cuda", fill=fill, kv_source=src)
    qs = [synth.normal_bf16(gd, (B, g.num_q_heads, g.head_dim)).cuda() for g in layers]
    kn = [synth.normal_bf16(gd, (B, g.num_kv_heads, g.head_dim)).cuda() for g in layers]
    vn = [None if g.k_eq_v else synth.normal_bf16(gd, (B, g.num_kv_heads, g.head_dim)).cuda()
          for g in layers]
    outs = [torch.empty((B, g.num_q_heads, g.head_dim), dtype=torch.float32, device="cuda")
            for g in layers]
    ctx_t = torch.from_numpy(ctx).cuda()
    pos = ctx_t - 1
    cache.step(qs, kn, vn, pos, ctx_t, pos, outs)
    torch.cuda.synchronize()
    for l, g in enumerate(layers):
        s = src[l]
        # the owner's slot of the newest token holds the owner's new row
        slot = (ctx - 1) % g.capacity if g.kind == api.RING else ctx - 1
        for b in range(B):
            assert torch.equal(cache.k[l][b, :, slot[b]], kn[s][b]), (l, b)
        inp = LayerInputs(synth.bits(qs[l]), synth.bits(cache.k[l]),
                          None if g.k_eq_v else synth.bits(cache.v[l]), ctx, ctx - 1)
        ref = oracle_out(inp, g.window, g.softcap, g.q_scale, g.kind)
        assert_parity(outs[l], ref, f"layer {l} (cache of {s})")


# ------------------------------------------------------------------ window / wrap alignment

@pytest.mark.parametrize("W", [64, 1024])
def test_window_and_wrap_alignments(W):
    """ctx around multiples of the window and of the split size: where other engines
    mis-selected sliding-window keys at particular seq_len/page alignments."""
    w = W
    ctxs = [1, w - 1, w, w + 1, 2 * w - 1, 2 * w, 2 * w + 1, 3 * w + 64, 5 * w - 63]
    geom = wl.sliding_geom(4, 2, w, softcap=50.0, scale=1.0 / 16)
    inp = layer_case(W, len(ctxs), geom, 1, 1, ctx=ctxs)
    ref = oracle_out(inp, w, geom.softcap, geom.q_scale, geom.kind)
    for split in [0, 64, 192, 1024]:
        out = run(inp, w, geom.softcap, geom.q_scale, geom.kind, split_keys=split,
                  max_ctx=max(ctxs))
        assert_parity(out, ref, f"W={W} split={split}")


def test_causal_query_below_newest_and_partial_window():
    """q_pos < ctx - 1 masks the later positions; windows narrower than the ring."""
    geom = wl.LayerGeom(8, 4, 256, api.RING, 256, 100, False, 0.0, 0.0625)
    inp = gen_layer(77, 6, 8, 4, 256, 256, False, 1, 1, ctx=[300, 300, 257, 256, 100, 5])
    inp.qpos = np.array([299, 250, 200, 255, 50, 0], np.int32)
    poison_invalid_slots(inp, geom.window, geom.kind, geom.capacity)
    inp.to_device()
    ref = oracle_out(inp, geom.window, 0.0, 0.0625, geom.kind)
    out = run(inp, geom.window, 0.0, 0.0625, geom.kind, max_ctx=300)
    assert_parity(out, ref, "causal/partial window")


def test_empty_rows_give_zero():
    geom = wl.global_geom(16, 512)
    inp = gen_layer(78, 3, 16, 1, 512, 512, True, 1, 1, ctx=[0, 10, 0]).to_device()
    for split in [0, 64]:
        out = run(inp, 0, 0.0, default_scale(512), api.LINEAR, split_keys=split)
        assert (out[0] == 0).all() and (out[2] == 0).all()
        assert torch.isfinite(out[1]).all() and out[1].abs().sum() > 0
    # the vector kernel's splits and the few-split merge (an empty row has no split to read;
    # the workspace is NaN-filled so any use of an unwritten partial would show)
    inp = gen_layer(78, 3, 4, 1, 256, 512, False, 1, 1, ctx=[0, 300, 0]).to_device()
    shape = api.shape_of(inp.q, inp.k, api.LINEAR, 512)
    for split in [64, 128]:
        nbytes = api.workspace_bytes(shape, 0, split_keys=split, impl=api.IMPL_VALU)
        assert nbytes > 0 and nbytes % 4 == 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ws.view(torch.float32).fill_(float("nan"))
        out = run(inp, 0, 0.0, default_scale(256), api.LINEAR, split_keys=split, max_ctx=512,
                  workspace=ws, impl=api.IMPL_VALU)
        assert (out[0] == 0).all() and (out[2] == 0).all(), split
        assert torch.isfinite(out[1]).all() and out[1].abs().sum() > 0, split
        ref = oracle_out(inp, 0, 0.0, default_scale(256), api.LINEAR)
        assert_parity(out, ref, f"empty rows, split {split}")


# ------------------------------------------------------------------ invariants

def test_constant_values_give_constant_output():
    """V = 1 everywhere: every softmax row sums to 1, so out = 1."""
    geom = wl.sliding_geom(16, 8, 1024)
    inp = gen_layer(79, 8, 16, 8, 256, 1024, False, 1, 5000)
    inp.v_bits[:] = 0x3F80
    inp.to_device()
    for split in [0, 64, 1024]:
        out = run(inp, 1024, 0.0, 1.0, api.RING, split_keys=split, max_ctx=5000)
        assert (out - 1.0).abs().max().item() < 1e-5


def test_single_valid_key_returns_that_row_bitwise():
    """ctx = 1, or window = 1: the output is that V row exactly."""
    inp = gen_layer(80, 4, 16, 8, 256, 64, False, 1, 1, ctx=[1, 40, 64, 200])
    inp.to_device()
    out = run(inp, 1, 50.0, 0.0625, api.RING, max_ctx=200)
    v = synth.from_bits(inp.v_bits, "cuda").float()
    for b, c in enumerate(inp.ctx):
        slot = (c - 1) % 64
        for h in range(16):
            assert torch.equal(out[b, h], v[b, h // 2, slot]), (b, h)


def test_split_count_invariance():
    g = wl.global_geom(16, 4096)
    inp = gen_layer(81, 4, 16, 1, 512, 4096, True, 100, 4096).to_device()
    base = run(inp, 0, 0.0, default_scale(512), api.LINEAR, split_keys=4096)
    for split in [64, 128, 448, 1024, 0]:
        out = run(inp, 0, 0.0, default_scale(512), api.LINEAR, split_keys=split,
                  impl=api.IMPL_VALU)
        max_abs, rel = errors(out, base.double().cpu().numpy())
        assert max_abs < 2e-5 and rel < 2e-5, (split, max_abs, rel)


def test_k_eq_v_null_equals_same_values_passed_twice():
    inp = gen_layer(82, 4, 16, 1, 512, 2048, True, 1, 2048).to_device()
    a = run(inp, 0, 0.0, default_scale(512), api.LINEAR, impl=api.IMPL_VALU, deterministic=True)
    copy = inp.k.clone()
    b = api.decode(inp.q, inp.k, copy, inp.ctx_t, inp.qpos_t, 0, 0.0, default_scale(512),
                   api.LINEAR, impl=api.IMPL_VALU, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_ring_equals_linear():
    """The same history in a ring and in a linear cache gives the same output: the same
    keys, summed in slot order on a full ring and in position order on the linear cache,
    so the two agree to within float32 rounding (bit for bit where the ring is not full)."""
    B, Hkv, D, W, total = 4, 2, 256, 128, 700
    gen = synth.generator(83)
    hist_k = synth.bits(synth.normal_bf16(gen, (B, Hkv, total, D)))
    hist_v = synth.bits(synth.normal_bf16(gen, (B, Hkv, total, D)))
    ring_k = np.full((B, Hkv, W, D), synth.BF16_NAN, np.uint16)
    ring_v = ring_k.copy()
    ctx = np.array([700, 555, 129, 100], np.int32)
    for b in range(B):
        for p in range(max(0, ctx[b] - W), ctx[b]):
            ring_k[b, :, p % W] = hist_k[b, :, p]
            ring_v[b, :, p % W] = hist_v[b, :, p]
    q = synth.normal_bf16(synth.generator(84), (B, 8, D)).cuda()
    ctx_t = torch.from_numpy(ctx).cuda()
    qp = ctx_t - 1
    a = api.decode(q, synth.from_bits(ring_k, "cuda"), synth.from_bits(ring_v, "cuda"), ctx_t, qp,
                   W, 0.0, 0.0625, api.RING, max_ctx=700, deterministic=True)
    b = api.decode(q, synth.from_bits(hist_k, "cuda"), synth.from_bits(hist_v, "cuda"), ctx_t, qp,
                   W, 0.0, 0.0625, api.LINEAR, deterministic=True)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    max_abs, rel = errors(a, b.double().cpu().numpy())
    assert max_abs < 2e-5 and rel < 2e-5, (max_abs, rel)
    assert torch.equal(a[3], b[3])  # ctx 100 < W: both layouts in position order


@pytest.mark.parametrize("geom", ["sliding", "global_valu"])
def test_deterministic_mode_repeats_bits_and_dynamic_agrees(geom):
    """With deterministic set, repeated calls give identical bits; the default (keys
    handed to waves as they free up) sums the same terms in another order, so it agrees
    to within a few float32 roundings."""
    if geom == "sliding":
        g = wl.sliding_geom(16, 8, 1024)
        inp = layer_case(86, 8, g, 1, 8192)
        kw = dict(max_ctx=8192)
    else:
        g = wl.global_geom(16, 6000)
        inp = layer_case(87, 4, g, 1000, 6000)
        kw = dict(impl=api.IMPL_VALU)
    args = (g.window, 0.0, g.q_scale, g.kind)
    d1 = run(inp, *args, deterministic=True, **kw)
    d2 = run(inp, *args, deterministic=True, **kw)
    assert torch.equal(d1, d2)
    for _ in range(3):
        dyn = run(inp, *args, **kw)
        max_abs, rel = errors(dyn, d1.double().cpu().numpy())
        assert max_abs < 2e-5 and rel < 2e-5, (max_abs, rel)


def test_gqa_equals_mha_with_repeated_kv():
    inp = gen_layer(85, 3, 8, 2, 256, 512, False, 100, 512).to_device()
    a = run(inp, 256, 0.0, 0.0625, api.RING, max_ctx=512)
    k_rep = inp.k.repeat_interleave(4, dim=1).contiguous()
    v_rep = inp.v.repeat_interleave(4, dim=1).contiguous()
    b = api.decode(inp.q, k_rep, v_rep, inp.ctx_t, inp.qpos_t, 256, 0.0, 0.0625, api.RING,
                   max_ctx=512)
    torch.cuda.synchronize()
    max_abs, rel = errors(a, b.double().cpu().numpy())
    assert max_abs < 1e-5 and rel < 1e-5


def test_violated_preconditions_stay_in_bounds_and_are_flagged():
    """q_pos >= ctx, ctx beyond max_ctx: the kernels clamp, outputs stay finite, and
    validate reports the rows."""
    geom = wl.sliding_geom(4, 2, 64)
    inp = gen_layer(86, 4, 4, 2, 256, 64, False, 1, 1, ctx=[10, 500, 64, 3])
    inp.qpos = np.array([20, 499, 63, 2], np.int32)
    inp.to_device()
    out = run(inp, 64, 0.0, 0.0625, api.RING, max_ctx=100)
    assert torch.isfinite(out).all()
    s = api.make_shape(4, 4, 2, 256, 64, api.RING, 100)
    flags = api.validate(s, inp.ctx_t, inp.qpos_t, 64).cpu().numpy()
    assert flags[0] & api.FLAG_QPOS_GE_CTX
    assert flags[1] & api.FLAG_OVER_MAX_CTX
    assert flags[2] == 0 and flags[3] == 0


def test_device_errors_launch_nothing():
    inp = gen_layer(87, 2, 4, 1, 256, 64, False, 10, 20).to_device()
    out = torch.full((2, 4, 256), 7.0, device="cuda")
    with pytest.raises(api.GemmaAttnError) as e:
        api.decode(inp.q, inp.k, inp.v, inp.ctx_t, inp.qpos_t, 65, 0.0, 0.0625, api.RING, out=out)
    assert e.value.code == -6
    with pytest.raises(api.GemmaAttnError) as e:
        api.decode(inp.q, inp.k, inp.v, inp.ctx_t, inp.qpos_t, 64, 0.0, math.nan, api.RING, out=out)
    assert e.value.code == -8
    torch.cuda.synchronize()
    assert (out == 7.0).all()


# ------------------------------------------------------------------ matrix-core global path

@pytest.mark.parametrize("case", ["one_long_row", "many_short_rows", "rows_at_grid_bound",
                                  "rows_past_grid_bound", "tile_edges", "ring_kv_shared"])
def test_mfma_partition_cases(case):
    """The matrix-core kernel cuts the batch's keys into equal chunks per work-group:
    one row spread over every work-group, hundreds of rows shorter than a tile, rows
    ending exactly on / next to tile and chunk edges, empty rows in between."""
    kind, cap, window, Hkv = api.LINEAR, 40000, 0, 1
    if case == "one_long_row":
        ctx = [40000]
    elif case == "many_short_rows":
        ctx = list(np.random.default_rng(90).integers(0, 40, size=600))
        cap = 64
    elif case == "rows_at_grid_bound":
        # 192 = 3/4 of the 256 work-groups (one per CU), all non-empty: the last unit count
        # for which the launch uses the plain grid; one work-group per row plus the rest
        ctx = list(np.random.default_rng(92).integers(1, 400, size=192))
        cap = 400
    elif case == "rows_past_grid_bound":
        # 193 non-empty rows: the grid grows by one work-group per unit
        ctx = list(np.random.default_rng(93).integers(1, 400, size=193))
        cap = 400
    elif case == "tile_edges":
        ctx = [16, 17, 15, 1, 0, 32, 4096, 4095, 4097, 0, 33, 1000]
        cap = 4097
    else:  # a ring cache, two KV heads of 16 query heads each
        kind, cap, window, Hkv = api.RING, 512, 300, 2
        ctx = [1, 299, 300, 301, 512, 513, 1500, 2047]
    B = len(ctx)
    inp = gen_layer(91, B, 16 * Hkv, Hkv, 512, cap, True, 1, 1, ctx=ctx)
    if B <= 64:
        poison_invalid_slots(inp, window, kind, cap)
    inp.to_device()
    max_ctx = cap if kind == api.LINEAR else max(ctx)
    scale = default_scale(512)
    out = run(inp, window, 0.0, scale, kind, impl=api.IMPL_MFMA, max_ctx=max_ctx)
    rows = list(range(B)) if B <= 64 else list(range(0, B, 7))
    ref = oracle_out(inp, window, 0.0, scale, kind, rows=rows)
    assert_parity(out[rows], ref, f"mfma {case}")
    empty = [b for b in range(B) if ctx[b] == 0]
    if empty:
        assert (out[empty] == 0).all()


def test_mfma_growing_logits_take_the_rescaling_path():
    """Logits that keep growing along the context (every key a larger multiple of q's
    direction): a wave's maximum rises far past its first step's, so the kernel leaves
    its fixed-reference loop for the rescaling one; rows of several lengths stop at
    different steps.  Against the oracle."""
    B, C = 4, 4096
    ctx = [4096, 3000, 1500, 700]
    inp = gen_layer(191, B, 16, 1, 512, C, True, 1, 1, ctx=ctx)
    # q = 1 in every head; key p = (p // 16) / 2 in every element (bf16-exact: at most 8
    # significant bits), so the scaled logit grows by 512 / 32 / sqrt(512) ~ 0.71 per
    # position (~1 log2 unit): a wave's steps 128 positions apart differ by ~130
    # (plus N(0, 1) noise per element, the sum rounded to bf16, so the values differ)
    inp.q_bits[:] = 0x3F80
    vals = ((np.arange(C) // 16) / 2.0).astype(np.float32)
    noise = torch.randn((B, 1, C, 512), generator=torch.Generator().manual_seed(7))
    grow = torch.from_numpy(vals)[None, None, :, None] + noise
    inp.k_bits[:] = synth.bits(grow.to(torch.bfloat16))
    bits = synth.bits((torch.from_numpy(vals[::-1].copy())[None, None, :, None] +
                       noise).to(torch.bfloat16))
    poison_invalid_slots(inp, 0, api.LINEAR, C)
    inp.to_device()
    scale = default_scale(512)
    ref = oracle_out(inp, 0, 0.0, scale, api.LINEAR)
    # balanced, and with long splits (1024 / 4096 keys: eight or more steps per wave)
    for split in [0, 1024, 4096]:
        out = run(inp, 0, 0.0, scale, api.LINEAR, split_keys=split, max_ctx=C)
        assert_parity(out, ref, f"growing logits split={split}")
    # decreasing logits stay on the fixed-reference loop: same check
    inp2 = gen_layer(192, B, 16, 1, 512, C, True, 1, 1, ctx=ctx)
    inp2.q_bits[:] = 0x3F80
    inp2.k_bits[:] = bits
    poison_invalid_slots(inp2, 0, api.LINEAR, C)
    inp2.to_device()
    ref2 = oracle_out(inp2, 0, 0.0, scale, api.LINEAR)
    for split in [0, 1024]:
        out = run(inp2, 0, 0.0, scale, api.LINEAR, split_keys=split, max_ctx=C)
        assert_parity(out, ref2, f"falling logits split={split}")


def test_mfma_more_units_than_one_launch():
    """B * Hkv = 2048 global-geometry units (more than the 1024 one launch takes): the
    library runs whole-row launches in stream order over one workspace, on the matrix
    cores.  NaN-poisoned slots, sampled rows against the oracle."""
    B, C = 2048, 256
    ctx = np.random.default_rng(94).integers(0, C + 1, size=B).astype(np.int32)
    ctx[:3] = [C, 1, 0]
    inp = gen_layer(193, B, 16, 1, 512, C, True, 1, 1, ctx=ctx)
    kb = inp.k_bits.reshape(B, C, 512)
    kb[np.arange(C)[None, :] >= ctx[:, None]] = synth.BF16_NAN  # never-valid slots
    inp.to_device()
    scale = default_scale(512)
    ws_auto = api.workspace_bytes(api.make_shape(B, 16, 1, 512, C, api.LINEAR), 0)
    out = run(inp, 0, 0.0, scale, api.LINEAR, max_ctx=C)
    assert torch.isfinite(out).all(), "a never-valid slot was read"
    rows = sorted({0, 1, 2, 1023, 1024, 1025, 2047} | set(range(5, B, 97)))
    ref = oracle_out(inp, 0, 0.0, scale, api.LINEAR, rows=rows)
    assert_parity(out[rows], ref, "2048 units")
    assert (out[2] == 0).all()
    # the same on the matrix cores explicitly, with a split size (fixed chunks per unit)
    out2 = run(inp, 0, 0.0, scale, api.LINEAR, max_ctx=C, split_keys=64, impl=api.IMPL_MFMA)
    assert_parity(out2[rows], ref, "2048 units, split 64")
    log(f"  workspace for the auto plan: {ws_auto} bytes")


def test_mfma_split_sizes_match_the_oracle():
    """A split size on the K = V global geometry keeps the matrix-core kernel (each unit in
    chunks of that many keys, merged by log-sum-exp): every size agrees with the oracle
    and with the balanced partition."""
    inp = gen_layer(194, 5, 16, 1, 512, 5000, True, 1, 1, ctx=[5000, 4097, 1, 0, 2500])
    poison_invalid_slots(inp, 0, api.LINEAR, 5000)
    inp.to_device()
    scale = default_scale(512)
    ref = oracle_out(inp, 0, 0.0, scale, api.LINEAR)
    base = run(inp, 0, 0.0, scale, api.LINEAR, impl=api.IMPL_MFMA)
    assert_parity(base, ref, "balanced")
    for split in [64, 128, 1024, 4096, 65536]:
        out = run(inp, 0, 0.0, scale, api.LINEAR, split_keys=split)
        assert_parity(out, ref, f"mfma split={split}")
        max_abs, rel = errors(out, base.double().cpu().numpy())
        assert max_abs < 1e-4 and rel < 1e-4, (split, max_abs, rel)


def test_mfma_matches_valu_and_softcap():
    inp = gen_layer(92, 8, 16, 1, 512, 3000, True, 1, 3000).to_device()
    scale = default_scale(512)
    for cap in [0.0, 30.0]:
        a = run(inp, 0, cap, scale, api.LINEAR, impl=api.IMPL_MFMA)
        b = run(inp, 0, cap, scale, api.LINEAR, impl=api.IMPL_VALU)
        max_abs, rel = errors(a, b.double().cpu().numpy())
        log(f"  mfma vs valu cap={cap}: max_abs={max_abs:.2e} rel={rel:.2e}")
        assert max_abs < 1e-4 and rel < 1e-4
    ref = oracle_out(inp, 0, 30.0, scale, api.LINEAR)
    assert_parity(run(inp, 0, 30.0, scale, api.LINEAR, impl=api.IMPL_MFMA), ref, "mfma softcap")


def test_mfma_repeats_bits_without_the_deterministic_option():
    """The global matrix-core kernel fixes its partition on the device from the context
    lengths and sums tiles, waves and work-groups in a fixed order: repeated calls give
    identical bits (bf16 and fp8 caches)."""
    inp = gen_layer(95, 6, 16, 1, 512, 9000, True, 1, 9000).to_device()
    scale = default_scale(512)
    a = run(inp, 0, 0.0, scale, api.LINEAR, impl=api.IMPL_MFMA)
    for _ in range(3):
        assert torch.equal(a, run(inp, 0, 0.0, scale, api.LINEAR, impl=api.IMPL_MFMA))
    codes = torch.randint(0, 126, (6, 1, 9000, 512), dtype=torch.uint8, device="cuda")
    scales = torch.rand((6, 1, 9000), device="cuda") * 0.01 + 0.001
    f = lambda: api.decode_fp8(inp.q, codes, scales, None, None, inp.ctx_t, inp.qpos_t, 0, 0.0,
                               scale, api.LINEAR, impl=api.IMPL_MFMA)
    b = f()
    for _ in range(3):
        assert torch.equal(b, f())


def test_mfma_single_key_rows_are_exact():
    """One valid key: P = 1 exactly splits into hi = 1, lo = 0, so the output is the row."""
    inp = gen_layer(93, 3, 16, 1, 512, 64, True, 1, 1, ctx=[1, 1, 1]).to_device()
    out = run(inp, 0, 0.0, default_scale(512), api.LINEAR, impl=api.IMPL_MFMA)
    k = synth.from_bits(inp.k_bits, "cuda").float()
    for b in range(3):
        for h in range(16):
            assert torch.equal(out[b, h], k[b, 0, 0])


# ------------------------------------------------------------------ fused append + decode

@pytest.mark.parametrize("case", ["sliding_ring", "sliding_split", "global_mfma", "global_valu",
                                  "ring_overwrites_valid", "positions_out_of_range"])
def test_decode_append_equals_append_then_decode(case):
    """One launch of gemma_attn_decode_append leaves the same cache bytes and the same
    output bits as gemma_kv_append followed by gemma_attn_decode."""
    rng = np.random.default_rng(hash(case) % 1000)
    impl, split, window = api.IMPL_AUTO, 0, 0
    if case in ("sliding_ring", "sliding_split", "ring_overwrites_valid"):
        B, Hq, Hkv, D, cap, kind, k_eq_v, window = 5, 16, 8, 256, 64, api.RING, False, 64
        ctx = np.array([1, 63, 64, 65, 300], np.int32)
        pos = ctx - 1
        if case == "sliding_split":
            split = 64
            cap, window = 256, 200
            ctx = np.array([1, 199, 200, 201, 900], np.int32)
            pos = ctx - 1
        if case == "ring_overwrites_valid":
            # appending position ctx (one past the context) overwrites the slot of ctx - W,
            # which is still valid: it must then read back as the new row
            pos = ctx.copy()
    elif case == "positions_out_of_range":
        B, Hq, Hkv, D, cap, kind, k_eq_v = 4, 16, 1, 512, 300, api.LINEAR, True
        ctx = np.array([10, 299, 300, 5], np.int32)
        pos = np.array([-1, 299, 300, 4], np.int32)  # -1 and C are skipped
    else:
        B, Hq, Hkv, D, cap, kind, k_eq_v = 6, 16, 1, 512, 3000, api.LINEAR, True
        ctx = np.array([1, 17, 1500, 2999, 3000, 700], np.int32)
        pos = ctx - 1
        impl = api.IMPL_MFMA if case == "global_mfma" else api.IMPL_VALU
    inp = gen_layer(94, B, Hq, Hkv, D, cap, k_eq_v, 1, 1, ctx=ctx).to_device()
    gen = synth.generator(95)
    k_new = synth.normal_bf16(gen, (B, Hkv, D)).cuda()
    v_new = None if k_eq_v else synth.normal_bf16(gen, (B, Hkv, D)).cuda()
    pos_t = torch.from_numpy(pos).cuda()
    max_ctx = int(ctx.max()) if kind == api.RING else cap
    scale = default_scale(D)
    # reference: append, then decode
    k1, v1 = inp.k.clone(), None if k_eq_v else inp.v.clone()
    api.kv_append(k1, v1, k_new, v_new, pos_t, kind)
    ref = api.decode(inp.q, k1, v1, inp.ctx_t, inp.qpos_t, window, 20.0, scale, kind,
                     max_ctx=max_ctx, split_keys=split, impl=impl, deterministic=True)
    # fused
    k2, v2 = inp.k.clone(), None if k_eq_v else inp.v.clone()
    got = api.decode_append(inp.q, k2, v2, k_new, v_new, pos_t, inp.ctx_t, inp.qpos_t, window,
                            20.0, scale, kind, max_ctx=max_ctx, split_keys=split, impl=impl,
                            deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)), "cache differs"
    if not k_eq_v:
        assert torch.equal(v1.view(torch.int16), v2.view(torch.int16)), "V cache differs"
    assert torch.isfinite(got).all()
    assert torch.equal(got, ref), (got - ref).abs().max().item()
    # and the result agrees with the oracle on the appended cache
    host = LayerInputs(inp.q_bits, synth.bits(k1), None if k_eq_v else synth.bits(v1), ctx,
                       inp.qpos)
    assert_parity(got, oracle_out(host, window, 20.0, scale, kind), f"decode_append {case}")


def test_binding_passes_a_small_workspace_to_the_library_which_refuses_it():
    """A caller-given workspace is not re-checked by the binding: the library compares it
    with what the plan needs and refuses a short one before launching anything (for the
    single-token, multi-token and fp8 entry points)."""
    B, Hq, Hkv, D, cap = 2, 16, 8, 256, 4096
    g = synth.generator(71, device="cuda")
    q = synth.normal_bf16(g, (B, Hq, D), "cuda")
    k = synth.normal_bf16(g, (B, Hkv, cap, D), "cuda")
    ctx = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    small = torch.empty((16,), dtype=torch.uint8, device="cuda")
    shape = api.shape_of(q, k, api.LINEAR, cap)
    assert api.workspace_bytes(shape, 0) > small.numel()  # 16 units over 8 splits
    with pytest.raises(api.GemmaAttnError) as e:
        api.decode(q, k, k, ctx, ctx - 1, 0, 0.0, default_scale(D), api.LINEAR,
                   workspace=small, max_ctx=cap)
    assert e.value.code == -7
    with pytest.raises(api.GemmaAttnError) as e:
        api.decode_multi(q[:, None].contiguous(), k, k, ctx, ctx - 1, 0, 0.0, default_scale(D),
                         api.LINEAR, workspace=small, max_ctx=cap)
    assert e.value.code == -7
    codes = torch.zeros((B, Hkv, cap, D), dtype=torch.uint8, device="cuda")
    scales = torch.ones((B, Hkv, cap), dtype=torch.float32, device="cuda")
    with pytest.raises(api.GemmaAttnError) as e:
        api.decode_fp8(q, codes, scales, codes, scales, ctx, ctx - 1, 0, 0.0, default_scale(D),
                       api.LINEAR, workspace=small, max_ctx=cap)
    assert e.value.code == -7
    torch.cuda.synchronize()
