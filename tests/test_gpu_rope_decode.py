"""GPU: RoPE + append + decode in one call equals RoPE + append followed by decode.

gemma_attn_decode_rope_append promises the bits of gemma_rope_append then
gemma_attn_decode_ex: the same rotated q, the same caches, the same output.  Where the
vector kernel serves the call, the rotation runs inside the decode launch (every
work-group rotates its unit's rows into LDS from the same per-element function); on
the global matrix-core kernel with a separate q_out too; for an in-place q_out with
several splits, and on the multi-token matrix-core kernel, the two calls run in turn.  Each case below runs both routes on copies of the same inputs and compares bit for
bit, and one case also checks the output against the oracle.
"""
import numpy as np
import pytest
import torch

from decode_attention_split_amd import api, synth

from common import LayerInputs, assert_parity, log, oracle_out

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, cap, kind, k_eq_v, ctx, seed):
    gen = synth.generator(seed)
    t = lambda shape: synth.normal_bf16(gen, shape).cuda()
    q = t((B, Hq, D))
    k = t((B, Hkv, cap, D))
    v = None if k_eq_v else t((B, Hkv, cap, D))
    kn = t((B, Hkv, D))
    vn = None if k_eq_v else t((B, Hkv, D))
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    return q, k, v, kn, vn, ctx_t


def _clone(x):
    return None if x is None else x.clone()


def _both_routes(q, k, v, kn, vn, ctx, window, softcap, scale, kind, base, R, in_place,
                 split_keys=0, impl=api.IMPL_AUTO, q_pos=None):
    pos = ctx - 1
    q_pos = pos if q_pos is None else q_pos
    # fused call
    kf, vf = k.clone(), _clone(v)
    qf = q.clone()
    qo = qf if in_place else torch.empty_like(q)
    table = api.rope_table(pos, base, R, q.shape[-1])
    out_f = api.decode_rope_append(qf, qo, kf, vf, kn, vn, pos, ctx, q_pos, window, softcap,
                                   scale, kind, table, R, split_keys=split_keys, impl=impl,
                                   deterministic=True)
    # the two calls
    kr, vr = k.clone(), _clone(v)
    qr = q.clone()
    qo_r = qr if in_place else torch.empty_like(q)
    api.rope_append(qr, qo_r, kr, vr, kn, vn, pos, kind, base, R)
    out_r = api.decode(qo_r, kr, vr, ctx, q_pos, window, softcap, scale, kind,
                       split_keys=split_keys, impl=impl, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(qo.view(torch.int16), qo_r.view(torch.int16)), "rotated q"
    assert torch.equal(kf.view(torch.int16), kr.view(torch.int16)), "k cache"
    if v is not None:
        assert torch.equal(vf.view(torch.int16), vr.view(torch.int16)), "v cache"
    assert torch.equal(out_f.view(torch.int32), out_r.view(torch.int32)), "output bits"
    return out_f, qo, kf, vf


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("split_keys", [0, 64])
def test_sliding_layer_fused_equals_two_calls(in_place, split_keys):
    """Gemma 3 / 4 sliding geometry: head_dim 256, 2 query heads per KV head, ring of the
    window; split_keys 64 gives four splits per row (fused with a separate q_out, the two
    calls with an in-place one); rows at an empty context, a partial ring, a wrapped ring."""
    B, Hq, Hkv, D, W = 5, 8, 4, 256, 256
    ctx = [0, 1, 100, 256, 9000]
    q, k, v, kn, vn, ctx_t = _case(B, Hq, Hkv, D, W, api.RING, False, ctx, 11 + split_keys)
    log(f"sliding rope decode: in_place={in_place} split_keys={split_keys}")
    _both_routes(q, k, v, kn, vn, ctx_t, W, 0.0, D ** -0.5, api.RING, 1e4, D, in_place,
                 split_keys=split_keys)


@pytest.mark.parametrize("D,Hq,Hkv,k_eq_v,R,kind,cap,window,softcap,impl", [
    (128, 8, 2, False, 64, api.LINEAR, 300, 0, 50.0, api.IMPL_AUTO),   # partial, 4 per KV
    (256, 4, 4, True, 256, api.RING, 32, 32, 0.0, api.IMPL_AUTO),      # K = V, vector kernel
    (512, 16, 1, True, 128, api.LINEAR, 2048, 0, 0.0, api.IMPL_AUTO),  # global: matrix cores
    (512, 16, 1, True, 128, api.LINEAR, 2048, 0, 30.0, api.IMPL_AUTO),  # the same, soft-capped
    (512, 16, 1, True, 128, api.LINEAR, 2048, 0, 0.0, api.IMPL_VALU),  # global: vector kernel
    (512, 2, 2, False, 512, api.RING, 64, 64, 30.0, api.IMPL_AUTO),    # one head per KV head
    (256, 16, 8, False, 0, api.RING, 128, 128, 0.0, api.IMPL_AUTO),    # no rotary part
])
def test_other_shapes_fused_equals_two_calls(D, Hq, Hkv, k_eq_v, R, kind, cap, window, softcap,
                                             impl):
    B = 4
    ctx = [1, cap // 2, cap, cap] if kind == api.LINEAR else [3, cap, 5 * cap + 7, 1]
    q, k, v, kn, vn, ctx_t = _case(B, Hq, Hkv, D, cap, kind, k_eq_v, ctx, D + Hq + R)
    log(f"rope decode D={D} Hq={Hq} Hkv={Hkv} K=V={k_eq_v} R={R} impl={impl}")
    base = 1e6 if D == 512 else 1e4
    for in_place in (False, True):
        _both_routes(q, k, v, kn, vn, ctx_t, window, softcap, D ** -0.5, kind, base, R,
                     in_place, impl=impl)


def test_global_fused_rows_without_keys_and_split_sizes():
    """The global geometry on the matrix cores with the rotation fused: rows with no valid
    key (an empty context, and q_pos = -1 with an append at position 4) have no work-group
    of their own, so work-group u writes their rotated q and appended row; the others
    several work-groups each.  Balanced over the chip and with split sizes 64 and 512."""
    B, Hq, Hkv, D, cap = 6, 16, 1, 512, 2048
    ctx = [0, 5, 1, 700, 2048, 1500]
    q, k, v, kn, vn, ctx_t = _case(B, Hq, Hkv, D, cap, api.LINEAR, True, ctx, 808)
    q_pos = ctx_t - 1
    q_pos[1] = -1
    for split in (0, 64, 512):
        log(f"global fused rope: split={split}")
        _both_routes(q, k, v, kn, vn, ctx_t, 0, 0.0, D ** -0.5, api.LINEAR, 1e6, 128, False,
                     split_keys=split, impl=api.IMPL_MFMA if split else api.IMPL_AUTO,
                     q_pos=q_pos)


def test_global_fused_more_units_than_one_launch():
    """1100 rows of one KV head: two matrix-core launches (at most 1024 units each) over
    one workspace, the rotation fused into both (the cos / sin table and q_out offset per
    launch)."""
    B, Hq, Hkv, D, cap = 1100, 16, 1, 512, 64
    gen = synth.generator(909)
    ctx = synth.uniform_int(gen, B, 1, cap).numpy().astype(np.int32).tolist()
    q, k, v, kn, vn, ctx_t = _case(B, Hq, Hkv, D, cap, api.LINEAR, True, ctx, 910)
    log("global fused rope: B=1100")
    _both_routes(q, k, v, kn, vn, ctx_t, 0, 0.0, D ** -0.5, api.LINEAR, 1e6, 128, False)


def test_fused_sliding_layer_matches_oracle():
    """The fused route against the oracle: rotate q and the new K row (the oracle's RoPE),
    append, attend."""
    import oracle
    B, Hq, Hkv, D, W = 3, 8, 4, 256, 256
    ctx = [2, 256, 700]
    q, k, v, kn, vn, ctx_t = _case(B, Hq, Hkv, D, W, api.RING, False, ctx, 5)
    kb, vb = synth.bits(k.cpu()), synth.bits(v.cpu())
    out, qo, kf, vf = _both_routes(q, k, v, kn, vn, ctx_t, W, 0.0, D ** -0.5, api.RING, 1e4, D,
                                   False, split_keys=64)
    pos = np.asarray(ctx, np.int64) - 1
    q_ref, _ = oracle.rope(synth.bits(q.cpu()), np.repeat(pos, Hq), 1e4, D)
    kn_ref, _ = oracle.rope(synth.bits(kn.cpu()), np.repeat(pos, Hkv), 1e4, D)
    k_ref, v_ref = kb.copy(), vb.copy()
    vnb = synth.bits(vn.cpu())
    for b in range(B):
        k_ref[b, :, pos[b] % W] = kn_ref[b]
        v_ref[b, :, pos[b] % W] = vnb[b]
    # rotation: same double arithmetic on both sides, at most rare one-ulp rounding ties
    diff = synth.bits(qo.cpu()).astype(np.int32) - q_ref.astype(np.int32)
    assert (np.abs(diff) <= 1).all() and (diff != 0).sum() <= 2
    diff = synth.bits(kf.cpu()).astype(np.int32) - k_ref.astype(np.int32)
    assert (np.abs(diff) <= 1).all() and (diff != 0).sum() <= 2
    assert np.array_equal(synth.bits(vf.cpu()), v_ref)
    ref = oracle_out(LayerInputs(q_ref, k_ref, v_ref, np.asarray(ctx, np.int32), pos), W, 0.0,
                     D ** -0.5, api.RING)
    assert_parity(out, ref, "fused rope decode")


def test_fused_call_rejects_bad_rotary_arguments():
    B, Hq, Hkv, D, W = 2, 4, 2, 128, 16
    q, k, v, kn, vn, ctx_t = _case(B, Hq, Hkv, D, W, api.RING, False, [3, 5], 3)
    pos = ctx_t - 1
    for R, base, hd in ((3, 1e4, D), (-2, 1e4, D), (D, 0.0, D), (D, float("inf"), D),
                        (D + 2, 1e4, D), (D, 1e4, 100), (D, 1e4, 0)):
        with pytest.raises(api.GemmaAttnError):
            api.rope_table(pos, base, R, hd)
    table = api.rope_table(pos, 1e4, D, D)
    for R in (3, D + 2, -2):
        with pytest.raises(api.GemmaAttnError):
            api.decode_rope_append(q, torch.empty_like(q), k, v, kn, vn, pos, ctx_t, pos, W,
                                   0.0, 1.0, api.RING, None, R)
    with pytest.raises(api.GemmaAttnError):  # no table for a rotary part
        api.decode_rope_append(q, torch.empty_like(q), k, v, kn, vn, pos, ctx_t, pos, W, 0.0,
                               1.0, api.RING, None, D)
    with pytest.raises(ValueError):  # a table of another rotary width
        api.decode_rope_append(q, torch.empty_like(q), k, v, kn, vn, pos, ctx_t, pos, W, 0.0,
                               1.0, api.RING, table, 64)


@pytest.mark.parametrize("base,R,D", [(1e4, 256, 256), (1e6, 128, 512), (1e4, 2, 128)])
def test_rope_table_matches_definition(base, R, D):
    """table[b, i] = (cos, sin) of pos[b] * base^(-2i/D) for the R/2 turning pairs, against
    numpy in double (angles up to about 1e5 radians lose a few digits to argument reduction
    on either side)."""
    pos = torch.tensor([0, 1, 255, 16383, 99999, -3], dtype=torch.int32, device="cuda")
    tab = api.rope_table(pos, base, R, D).cpu().numpy()
    i = np.arange(R // 2)
    ang = pos.cpu().numpy().astype(np.float64)[:, None] * np.power(float(base), -2.0 * i / D)
    assert tab.shape == (6, R // 2, 2)
    np.testing.assert_allclose(tab[..., 0], np.cos(ang), rtol=0, atol=1e-10)
    np.testing.assert_allclose(tab[..., 1], np.sin(ang), rtol=0, atol=1e-10)
    assert (tab[0, :, 0] == 1.0).all() and (tab[0, :, 1] == 0.0).all()


@pytest.mark.parametrize("layer", [0, 5])
def test_rope_step_layer_full_size_sampled_rows(layer):
    """The 48-layer RoPE step's layers at full size, in the launch the bench times (one
    call per layer on the step's cos / sin table): sliding layer 0 and global layer 5 (matrix
    cores), each one launch, sampled rows against the oracle's rotate, append, attend."""
    from decode_attention_split_amd import workloads as wl
    from common import gen_layer
    import oracle
    w = wl.HYBRID_48_ROPE
    g = w.layers[layer]
    log(f"rope step layer {layer}: {'global' if g.k_eq_v else 'sliding'} R={g.rotary_dim}")
    inp = gen_layer(wl.layer_seed(w, layer), w.batch, g.num_q_heads, g.num_kv_heads,
                    g.head_dim, g.capacity, g.k_eq_v, w.ctx_lo, w.ctx_hi).to_device()
    gen = synth.generator(1000 + layer)
    kn = synth.normal_bf16(gen, (w.batch, g.num_kv_heads, g.head_dim))
    vn = None if g.k_eq_v else synth.normal_bf16(gen, (w.batch, g.num_kv_heads, g.head_dim))
    pos_t = inp.ctx_t - 1
    max_ctx = min(w.ctx_hi, g.capacity) if g.kind == api.LINEAR else w.ctx_hi
    table = api.rope_table(pos_t, g.rope_base, g.rotary_dim, g.head_dim)
    q_out = torch.empty_like(inp.q)
    out = api.decode_rope_append(inp.q, q_out, inp.k, inp.v, kn.cuda(),
                                 None if vn is None else vn.cuda(), pos_t, inp.ctx_t, pos_t,
                                 g.window, g.softcap, g.q_scale, g.kind, table, g.rotary_dim,
                                 max_ctx=max_ctx)
    torch.cuda.synchronize()
    rows = sorted({0, 7, int(np.argmax(inp.ctx)), int(np.argmin(inp.ctx))})
    pos = inp.ctx[rows].astype(np.int64) - 1
    q_ref, _ = oracle.rope(inp.q_bits[rows], np.repeat(pos, g.num_q_heads), g.rope_base,
                           g.rotary_dim)
    kn_ref, _ = oracle.rope(synth.bits(kn)[rows], np.repeat(pos, g.num_kv_heads), g.rope_base,
                            g.rotary_dim)
    k_ref = inp.k_bits[rows].copy()
    v_ref = None if vn is None else inp.v_bits[rows].copy()
    for i, p in enumerate(pos):
        s = p % g.capacity if g.kind == api.RING else p
        k_ref[i, :, s] = kn_ref[i]
        if v_ref is not None:
            v_ref[i, :, s] = synth.bits(vn)[rows[i]]
    diff = synth.bits(q_out.cpu())[rows].astype(np.int32) - q_ref.astype(np.int32)
    assert (np.abs(diff) <= 1).all() and (diff != 0).sum() <= max(2, diff.size // 10000)
    ref = oracle_out(LayerInputs(q_ref, k_ref, v_ref, inp.ctx[rows], pos), g.window, g.softcap,
                     g.q_scale, g.kind)
    assert_parity(out[rows], ref, f"rope step layer {layer} rows {rows}")
