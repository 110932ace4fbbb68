"""GPU: rotary embedding fused with the cache append, against the oracle.

Both sides compute the rotation in double and round once to bf16 (nearest, ties to even),
so the bits agree except where the two double results straddle a bf16 rounding tie (their
sin/cos agree to about one double ulp): the tests allow at most a handful of elements to
differ, each by one bf16 ulp, and require everything else to match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_split_amd import api, synth
from decode_attention_split_amd import workloads as wl
from decode_attention_split_amd.hybrid import HybridKVCache

from common import LayerInputs, assert_parity, log, oracle_out

pytestmark = pytest.mark.gpu


def assert_bits_close(got, ref, what):
    got = np.asarray(got, np.uint16).astype(np.int32)
    ref = np.asarray(ref, np.uint16).astype(np.int32)
    diff = got != ref
    n_diff = int(diff.sum())
    # same sign, adjacent codes (one bf16 ulp)
    assert (np.abs(got[diff] - ref[diff]) == 1).all(), f"{what}: difference beyond one ulp"
    assert n_diff <= max(2, got.size // 10000), f"{what}: {n_diff} of {got.size} differ"
    if n_diff:
        log(f"  {what}: {n_diff} of {got.size} elements one ulp apart")


def expected(q_bits, k_bits, v_bits, kn_bits, vn_bits, pos0, kind, base, R):
    B, T, Hq, D = q_bits.shape
    Hkv, cap = k_bits.shape[1], k_bits.shape[2]
    qpos = np.repeat((pos0[:, None] + np.arange(T)[None, :]).reshape(-1), Hq)
    q_ref, _ = oracle.rope(q_bits, qpos, base, R)
    kpos = np.repeat((pos0[:, None] + np.arange(T)[None, :]).reshape(-1), Hkv)
    kn_rot, _ = oracle.rope(kn_bits, kpos, base, R)
    k_ref, v_ref = k_bits.copy(), None if v_bits is None else v_bits.copy()
    for b in range(B):
        for t in range(T):  # in order: a later token owns a shared ring slot
            p = int(pos0[b]) + t
            if p < 0 or (kind == api.LINEAR and p >= cap):
                continue
            s = p % cap if kind == api.RING else p
            k_ref[b, :, s] = kn_rot[b, t]
            if v_ref is not None:
                v_ref[b, :, s] = vn_bits[b, t]
    return q_ref, k_ref, v_ref


@pytest.mark.parametrize("D,R,base,kind,k_eq_v,T,cap,pos0", [
    (256, 256, 1e4, api.RING, False, 1, 64, [0, 63, 64, 9000]),            # sliding layer
    (512, 128, 1e6, api.LINEAR, True, 1, 40000, [0, 17, 32767, 39999]),    # global, partial
    (128, 64, 1e4, api.RING, False, 4, 32, [0, 30, 100, 5]),
    (256, 256, 1e4, api.RING, False, 6, 4, [0, 7, 13, 2]),                 # T > W: wraps
    (256, 96, 1e4, api.LINEAR, False, 3, 16, [-2, 5, 14, 0]),             # skipped positions
    (512, 0, 1e6, api.LINEAR, True, 2, 64, [1, 2, 3, 4]),                  # no rotary part
])
def test_rope_append_matches_oracle(D, R, base, kind, k_eq_v, T, cap, pos0):
    B, Hq, Hkv = 4, 8, 2
    gen = synth.generator(D + R + T)
    q = synth.normal_bf16(gen, (B, T, Hq, D))
    k = synth.normal_bf16(gen, (B, Hkv, cap, D))
    v = None if k_eq_v else synth.normal_bf16(gen, (B, Hkv, cap, D))
    kn = synth.normal_bf16(gen, (B, T, Hkv, D))
    vn = None if k_eq_v else synth.normal_bf16(gen, (B, T, Hkv, D))
    pos0 = np.asarray(pos0, np.int32)
    q_ref, k_ref, v_ref = expected(synth.bits(q), synth.bits(k), None if v is None else
                                   synth.bits(v), synth.bits(kn), None if vn is None else
                                   synth.bits(vn), pos0, kind, base, R)
    qd, kd = q.cuda(), k.cuda()
    vd = None if v is None else v.cuda()
    q_out = torch.empty_like(qd)
    api.rope_append(qd, q_out, kd, vd, kn.cuda(), None if vn is None else vn.cuda(),
                    torch.from_numpy(pos0).cuda(), kind, base, R)
    torch.cuda.synchronize()
    assert_bits_close(synth.bits(q_out.cpu()), q_ref, "q")
    assert_bits_close(synth.bits(kd.cpu()), k_ref, "k cache")
    if v is not None:
        assert np.array_equal(synth.bits(vd.cpu()), v_ref), "v cache (unrotated copy)"
    # in place: q_out aliasing q gives the same bits
    api.rope_append(qd, qd, kd, vd, kn.cuda(), None if vn is None else vn.cuda(),
                    torch.from_numpy(pos0).cuda(), kind, base, R)
    torch.cuda.synchronize()
    assert torch.equal(qd, q_out)


def test_hybrid_step_with_rope_matches_oracle():
    """A 12-layer stack (sliding base 1e4 over the whole head, global base 1e6 over a
    quarter of it, last 4 layers sharing caches): one step of rotary + append + decode per
    layer equals the oracle's rotate, append, attend on every layer."""
    sl = wl.with_rope(wl.sliding_geom(8, 4, 128), 1e4, 256)
    gl = wl.with_rope(wl.global_geom(16, 1024), 1e6, 128)
    layers = wl.hybrid_layers(12, sl, gl)
    src = wl.kv_share_sources(layers, 4)
    B = 3
    ctx = np.array([1, 300, 1024], np.int32)
    gd = synth.generator(97)
    fill = lambda li, name, shape: synth.normal_bf16(gd, shape).cuda()
    cache = HybridKVCache(layers, B, 1024, device="cuda", fill=fill, kv_source=src)
    k0 = [synth.bits(t.cpu()) for t in cache.k]
    v0 = [None if t is None else synth.bits(t.cpu()) for t in cache.v]
    qs = [synth.normal_bf16(gd, (B, g.num_q_heads, g.head_dim)).cuda() for g in layers]
    kn = [synth.normal_bf16(gd, (B, g.num_kv_heads, g.head_dim)).cuda() for g in layers]
    vn = [None if g.k_eq_v else synth.normal_bf16(gd, (B, g.num_kv_heads, g.head_dim)).cuda()
          for g in layers]
    outs = [torch.empty((B, g.num_q_heads, g.head_dim), dtype=torch.float32, device="cuda")
            for g in layers]
    q_rot = [torch.empty_like(q) for q in qs]
    ctx_t = torch.from_numpy(ctx).cuda()
    pos = ctx_t - 1
    cache.step(qs, kn, vn, pos, ctx_t, pos, outs, q_rot=q_rot)
    torch.cuda.synchronize()
    # oracle: the owner layers' caches after their rotated appends
    ref_k, ref_v = {}, {}
    for l, g in enumerate(layers):
        if src[l] != l:
            continue
        qb = synth.bits(qs[l].cpu())[:, None]
        _, kr, vr = expected(qb, k0[l], v0[l], synth.bits(kn[l].cpu())[:, None],
                             None if vn[l] is None else synth.bits(vn[l].cpu())[:, None],
                             ctx - 1, g.kind, g.rope_base, g.rotary_dim)
        ref_k[l], ref_v[l] = kr, vr
    for l, g in enumerate(layers):
        q_ref, _ = oracle.rope(synth.bits(qs[l].cpu()), np.repeat(ctx - 1, g.num_q_heads),
                               g.rope_base, g.rotary_dim)
        assert_bits_close(synth.bits(q_rot[l].cpu()), q_ref, f"layer {l} q")
        s = src[l]
        assert_bits_close(synth.bits(cache.k[l].cpu()), ref_k[s], f"layer {l} k cache")
        inp = LayerInputs(q_ref, ref_k[s], ref_v[s], ctx, ctx - 1)
        ref = oracle_out(inp, g.window, g.softcap, g.q_scale, g.kind)
        assert_parity(outs[l], ref, f"rope layer {l}")
