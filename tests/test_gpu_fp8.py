"""GPU: fp8 e4m3 caches (codes + per-row float32 scales): the quantizing append bit for
bit, and decode (one or several query tokens) against the fp64 oracle over the same codes.

Parity cases poison every slot outside the valid set: codes 0x7f (NaN) and scale NaN, so
a stray read turns the output NaN.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_split_amd import api, synth
from decode_attention_split_amd import workloads as wl

from common import assert_parity, default_scale, errors, f32, log

pytestmark = pytest.mark.gpu

FP8_NAN = 0x7F


class Fp8Inputs:
    """Random finite codes and positive row scales (host copies) and device tensors."""

    def __init__(self, seed, B, T, Hq, Hkv, D, cap, k_eq_v, ctx, q0=None):
        rng = np.random.default_rng(seed)
        finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
        gen = synth.generator(seed)
        self.q_bits = synth.bits(synth.normal_bf16(gen, (B, T, Hq, D)))
        self.kc = rng.choice(finite, size=(B, Hkv, cap, D))
        self.ks = rng.uniform(0.002, 0.02, (B, Hkv, cap)).astype(np.float32)
        self.vc = None if k_eq_v else rng.choice(finite, size=(B, Hkv, cap, D))
        self.vs = None if k_eq_v else rng.uniform(0.002, 0.02, (B, Hkv, cap)).astype(np.float32)
        self.ctx = np.asarray(ctx, np.int32)
        self.q0 = self.ctx - T if q0 is None else np.asarray(q0, np.int32)
        self.T, self.cap = T, cap

    def poison(self, window, kind):
        for c, sc in [(self.kc, self.ks)] + ([(self.vc, self.vs)] if self.vc is not None else []):
            for b in range(c.shape[0]):
                keep = np.zeros(self.cap, bool)
                for t in range(self.T):
                    _, slots = oracle.valid_positions(self.ctx[b], self.q0[b] + t, window, kind,
                                                      self.cap)
                    keep[slots] = True
                c[b][:, ~keep, :] = FP8_NAN
                sc[b][:, ~keep] = np.nan
        return self

    def to_device(self):
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.q = synth.from_bits(self.q_bits, "cuda")
        self.kc_d, self.ks_d, self.vc_d, self.vs_d = t(self.kc), t(self.ks), t(self.vc), t(self.vs)
        self.ctx_t, self.q0_t = t(self.ctx), t(self.q0)
        return self

    def oracle(self, window, softcap, scale, kind, rows=None):
        rows = np.arange(self.q_bits.shape[0]) if rows is None else np.asarray(rows)
        pick = lambda a: None if a is None else a[rows]
        out, _, _, flags = oracle.decode_fp8_multi(
            self.q_bits[rows], self.kc[rows], self.ks[rows], pick(self.vc), pick(self.vs),
            self.ctx[rows], self.q0[rows], window, softcap, scale, kind)
        return out, flags

    def run(self, window, softcap, scale, kind, **kw):
        q = self.q[:, 0].contiguous() if self.T == 1 else self.q
        out = api.decode_fp8(q, self.kc_d, self.ks_d, self.vc_d, self.vs_d, self.ctx_t, self.q0_t,
                             window, softcap, scale, kind, **kw)
        torch.cuda.synchronize()
        return out.unsqueeze(1) if self.T == 1 else out


@pytest.mark.parametrize("D", [128, 256, 512])
@pytest.mark.parametrize("k_eq_v", [False, True])
@pytest.mark.parametrize("T", [1, 4, 12])  # 12 > the ring's 8 slots: later tokens own them
def test_append_fp8_matches_oracle_bitwise(D, k_eq_v, T):
    B, Hkv = 3, 2
    for kind, cap, pos0 in [(api.RING, 8, [0, 5, 1001]), (api.LINEAR, 16, [-2, 3, 14])]:
        gen = synth.generator(D + T + kind)
        kn = synth.normal_bf16(gen, (B, T, Hkv, D)) * 3
        kn[0, 0, 0] = 0  # an all-zero row: codes 0, scale 0
        vn = None if k_eq_v else synth.normal_bf16(gen, (B, T, Hkv, D))
        kc = np.full((B, Hkv, cap, D), 0x11, np.uint8)
        ks = np.full((B, Hkv, cap), 7.0, np.float32)
        vc, vs = (None, None) if k_eq_v else (kc.copy(), ks.copy())
        dev = [None if a is None else torch.from_numpy(a.copy()).cuda() for a in (kc, ks, vc, vs)]
        api.kv_append_fp8(dev[0], dev[1], dev[2], dev[3], kn.cuda(),
                          None if vn is None else vn.cuda(),
                          torch.tensor(pos0, dtype=torch.int32, device="cuda"), kind)
        torch.cuda.synchronize()
        oracle.append_fp8(kc, ks, synth.bits(kn), np.asarray(pos0, np.int32), kind)
        assert np.array_equal(dev[0].cpu().numpy(), kc), (kind, "K codes")
        assert np.array_equal(dev[1].cpu().numpy().view(np.uint32), ks.view(np.uint32)), \
            (kind, "K scales")
        if not k_eq_v:
            oracle.append_fp8(vc, vs, synth.bits(vn), np.asarray(pos0, np.int32), kind)
            assert np.array_equal(dev[2].cpu().numpy(), vc), (kind, "V codes")
            assert np.array_equal(dev[3].cpu().numpy().view(np.uint32), vs.view(np.uint32))


@pytest.mark.parametrize("D,G,Hkv", [(128, 4, 2), (256, 1, 2), (256, 2, 4), (256, 8, 1),
                                     (512, 2, 1), (512, 16, 1)])
@pytest.mark.parametrize("kind", [api.RING, api.LINEAR])
@pytest.mark.parametrize("T", [1, 3])
def test_fp8_decode_parity_sweep(D, G, Hkv, kind, T):
    w = 100
    if kind == api.RING:
        cap, window = w + T - 1, w
        ctx = [1, 37, w, w + 1, 5 * cap + 3]
        max_ctx = max(ctx)
    else:
        cap, window = 500, (w if G <= 2 else 0)
        ctx = [1, 37, 300, 499, 500]
        max_ctx = cap
    inp = Fp8Inputs(D + 10 * G + 100 * T + kind, len(ctx), T, G * Hkv, Hkv, D, cap, G == 16, ctx)
    inp.poison(window, kind).to_device()
    softcap = 30.0 if G % 2 == 0 else 0.0
    ref, _ = inp.oracle(window, softcap, default_scale(D), kind)
    for split in [0, 64]:
        out = inp.run(window, softcap, default_scale(D), kind, max_ctx=max_ctx, split_keys=split)
        assert_parity(out, ref, f"fp8 D={D} G={G} kind={kind} T={T} split={split}")


def test_fp8_spec_decode_window_edges():
    """BF16 queries, FP8 cache, 8 query tokens on a sliding window: the combination that
    mis-selected window keys at some seq_len alignments in another engine."""
    T, w = 8, 64
    cap = w + T - 1
    ctxs = [T, w - 1, w, w + 1, w + T - 1, 2 * w, 2 * w + 3, 3 * w + T, 5 * w - 1]
    inp = Fp8Inputs(55, len(ctxs), T, 16, 8, 256, cap, False, ctxs)
    inp.poison(w, api.RING).to_device()
    ref, flags = inp.oracle(w, 50.0, 1.0 / 16, api.RING)
    assert not flags.any()
    for split in [0, 64]:
        out = inp.run(w, 50.0, 1.0 / 16, api.RING, max_ctx=max(ctxs), split_keys=split)
        assert_parity(out, ref, f"fp8 spec split={split}")


def test_fp8_equals_bf16_kernel_on_exactly_representable_values():
    """With power-of-two row scales every code * scale is a bf16 value: the fp8 and bf16
    kernels then see the same numbers (rounding order aside)."""
    B, Hq, Hkv, D, cap = 4, 16, 8, 256, 256
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    kc = rng.choice(finite, size=(B, Hkv, cap, D))
    vc = rng.choice(finite, size=(B, Hkv, cap, D))
    ks = np.ldexp(1.0, rng.integers(-8, -3, (B, Hkv, cap))).astype(np.float32)
    vs = np.ldexp(1.0, rng.integers(-8, -3, (B, Hkv, cap))).astype(np.float32)
    tv = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).float()
    kb = (tv(kc) * torch.from_numpy(ks)[..., None]).to(torch.bfloat16).cuda()
    vb = (tv(vc) * torch.from_numpy(vs)[..., None]).to(torch.bfloat16).cuda()
    q = synth.normal_bf16(synth.generator(6), (B, Hq, D)).cuda()
    ctx = torch.tensor([1, 100, 255, 256], dtype=torch.int32, device="cuda")
    a = api.decode_fp8(q, torch.from_numpy(kc).cuda(), torch.from_numpy(ks).cuda(),
                       torch.from_numpy(vc).cuda(), torch.from_numpy(vs).cuda(), ctx, ctx - 1, 0,
                       0.0, 0.0625, api.LINEAR)
    b = api.decode(q, kb, vb, ctx, ctx - 1, 0, 0.0, 0.0625, api.LINEAR)
    torch.cuda.synchronize()
    max_abs, rel = errors(a, b.double().cpu().numpy())
    # two float32 sums of the same terms in different orders; outputs reach ~30 in size
    assert max_abs < 1e-4 and rel < 1e-5, (max_abs, rel)


def test_fp8_sliding_layer_full_size_sampled_rows():
    """The 12B sliding-layer geometry (B 64, 16q/8kv, hd256, ring W = w = 1024, ctx
    U[512, 8192], soft-cap 50) on an fp8 cache filled by one quantizing append of 1024
    tokens per row; sampled rows checked against the oracle (codes and outputs)."""
    w = wl.G4_12B_SLIDING
    g = w.layers[0]
    B, Hkv, D, W = w.batch, g.num_kv_heads, g.head_dim, g.capacity
    ctx = synth.uniform_int(synth.generator(w.seed), B, w.ctx_lo, w.ctx_hi).numpy() \
        .astype(np.int32)
    gd = synth.generator(77, device="cuda")
    kc = torch.empty((B, Hkv, W, D), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    ks = torch.empty((B, Hkv, W), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    ctx_t = torch.from_numpy(ctx).cuda()
    pos0 = ctx_t - W  # the newest W positions of every row
    kn = synth.normal_bf16(gd, (B, W, Hkv, D), device="cuda")
    vn = synth.normal_bf16(gd, (B, W, Hkv, D), device="cuda")
    api.kv_append_fp8(kc, ks, vc, vs, kn, vn, pos0, api.RING)
    q = synth.normal_bf16(gd, (B, g.num_q_heads, D), device="cuda")
    out = api.decode_fp8(q, kc, ks, vc, vs, ctx_t, ctx_t - 1, g.window, g.softcap, g.q_scale,
                         g.kind, max_ctx=w.ctx_hi)
    torch.cuda.synchronize()
    rows = sorted({0, 1, int(np.argmax(ctx)), int(np.argmin(ctx))})
    log(f"fp8 sliding rows {rows}")
    kcr, ksr = kc[rows].cpu().numpy(), ks[rows].cpu().numpy()
    vcr, vsr = vc[rows].cpu().numpy(), vs[rows].cpu().numpy()
    # the cache holds exactly the oracle's quantization of the appended rows
    for i, b in enumerate(rows):
        for t in (0, 517, W - 1):
            if int(ctx[b]) - W + t < 0:
                continue  # negative positions are skipped by the append
            slot = (int(ctx[b]) - W + t) % W
            c, s = oracle.quantize_rows_fp8(synth.bits(kn[b, t].cpu()))
            assert np.array_equal(kcr[i, :, slot], c) and np.array_equal(ksr[i, :, slot], s)
    ref, _, _, _ = oracle.decode_fp8_multi(synth.bits(q[rows].cpu()), kcr, ksr, vcr, vsr,
                                           ctx[rows], ctx[rows] - 1, g.window, g.softcap,
                                           g.q_scale, g.kind)
    assert_parity(out[rows], ref, "fp8 sliding full size")


@pytest.mark.parametrize("kind", [api.RING, api.LINEAR])
def test_fp8_global_matrix_cores_match_vector_kernel_and_oracle(kind):
    """The K = V global geometry (hd512, 16 query heads per KV head) on fp8 codes: the
    matrix-core kernel (codes widened to bf16 in registers, scales on logits and value
    weights) and the vector kernel both match the oracle, over ragged contexts that leave
    partial 16-key tiles, a one-key row and rows split over several work-groups."""
    Hkv, D = 2, 512
    if kind == api.RING:
        cap, window = 300, 300
        ctx = [1, 16, 17, 299, 300, 1000, 4 * 300 + 7]
        max_ctx = max(ctx)
    else:
        cap, window = 700, 0
        ctx = [1, 16, 17, 333, 512, 699, 700]
        max_ctx = cap
    inp = Fp8Inputs(4242 + kind, len(ctx), 1, 16 * Hkv, Hkv, D, cap, True, ctx)
    inp.poison(window, kind).to_device()
    for softcap in [0.0, 30.0]:
        ref, _ = inp.oracle(window, softcap, default_scale(D), kind)
        for impl in [api.IMPL_MFMA, api.IMPL_VALU]:
            out = inp.run(window, softcap, default_scale(D), kind, max_ctx=max_ctx, impl=impl)
            assert_parity(out, ref, f"fp8 global kind={kind} softcap={softcap} impl={impl}")


@pytest.mark.parametrize("s_lo,s_hi,q_pow2", [
    (1e-7, 2e-7, 0),    # quiet rows: p * s far below fp16's normal range unless normalized
    (50.0, 400.0, 0),   # loud rows: p * s * 448 far beyond fp16's range unless normalized
    (1e-4, 0.4, 0),     # row scales spanning 2^12 inside one unit
    (0.002, 0.02, 16),  # |q| up to ~2^18: beyond fp16's range unless normalized
    (0.002, 0.02, -24),  # |q| ~ 2^-24: fp16 subnormals unless normalized
])
def test_fp8_global_matrix_cores_extreme_ranges(s_lo, s_hi, q_pow2):
    """The matrix-core fp8 path multiplies in fp16 (exact for e4m3 codes) and keeps q and
    the value weights p * s in fp16's range with powers of two per work-group; row scales
    and query magnitudes far from 1 must still match the oracle.  The attention scale keeps
    the logits near unit size (scaled q comes with the inverse scale, an exact power of
    two), and both outputs are divided by the largest reference value before the usual
    tolerances apply, since those are absolute."""
    Hkv, D, cap = 1, 512, 4096
    ctx = [1, 700, 2500, 4096]
    inp = Fp8Inputs(777, len(ctx), 1, 16, Hkv, D, cap, True, ctx)
    rng = np.random.default_rng(778)
    inp.ks = np.exp(rng.uniform(np.log(s_lo), np.log(s_hi), inp.ks.shape)).astype(np.float32)
    att = f32(1.0 / (math.sqrt(D) * 120.0 * math.sqrt(s_lo * s_hi)))
    if q_pow2:
        q = synth.from_bits(inp.q_bits, "cpu").float() * 2.0 ** q_pow2
        inp.q_bits = synth.bits(q.to(torch.bfloat16))
        att = f32(att * 2.0 ** -q_pow2)
    inp.to_device()
    ref, _ = inp.oracle(0, 0.0, att, api.LINEAR)
    out = inp.run(0, 0.0, att, api.LINEAR, max_ctx=cap, impl=api.IMPL_MFMA)
    big = float(np.abs(ref).max())
    assert big > 0
    assert_parity(out.double().cpu().numpy() / big, ref / big,
                  f"fp8 global extreme ranges s=[{s_lo}, {s_hi}] q*2^{q_pow2}")


@pytest.mark.parametrize("s_lo,s_hi,q_pow2", [
    (1e-7, 2e-7, 0), (50.0, 400.0, 0), (1e-4, 0.4, 0), (0.002, 0.02, 16), (0.002, 0.02, -24),
])
def test_fp8_multi_token_matrix_cores_extreme_ranges(s_lo, s_hi, q_pow2):
    """The multi-token matrix-core fp8 path (16 query rows per KV head: 2 heads x 8 tokens,
    separate K and V): K and V row scales and query magnitudes far from 1 must still match
    the oracle (compared after dividing by the largest reference value)."""
    B, T, Hq, Hkv, D, cap = 3, 8, 4, 2, 256, 300
    ctx = [9, 150, 300]
    inp = Fp8Inputs(779, B, T, Hq, Hkv, D, cap, False, ctx)
    rng = np.random.default_rng(780)
    draw = lambda shape: np.exp(rng.uniform(np.log(s_lo), np.log(s_hi), shape)).astype(np.float32)
    inp.ks, inp.vs = draw(inp.ks.shape), draw(inp.vs.shape)
    att = f32(1.0 / (math.sqrt(D) * 120.0 * math.sqrt(s_lo * s_hi)))
    if q_pow2:
        q = synth.from_bits(inp.q_bits, "cpu").float() * 2.0 ** q_pow2
        inp.q_bits = synth.bits(q.to(torch.bfloat16))
        att = f32(att * 2.0 ** -q_pow2)
    inp.to_device()
    ref, _ = inp.oracle(0, 0.0, att, api.LINEAR)
    out = inp.run(0, 0.0, att, api.LINEAR, max_ctx=cap, impl=api.IMPL_MFMA)
    big = float(np.abs(ref).max())
    assert big > 0
    assert_parity(out.double().cpu().numpy() / big, ref / big,
                  f"fp8 multi-token extreme ranges s=[{s_lo}, {s_hi}] q*2^{q_pow2}")


def test_fp8_global_layer_full_size_sampled_rows():
    """The 12B global layer (B 16, 16q/1kv K = V hd512, linear C 32768, ctx U[4096, 32768])
    on an fp8 cache filled by quantizing appends of every valid position; the automatic
    plan (matrix cores) checked against the oracle on sampled rows."""
    w = wl.FP8_GLOBAL
    g = w.layers[0]
    B, D, C = w.batch, g.head_dim, g.capacity
    ctx = synth.uniform_int(synth.generator(w.seed), B, w.ctx_lo, w.ctx_hi).numpy() \
        .astype(np.int32)
    gd = synth.generator(91, device="cuda")
    kc = torch.empty((B, 1, C, D), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, 1, C), dtype=torch.float32, device="cuda")
    chunk = 1024
    for p0 in range(0, int(ctx.max()), chunk):
        kn = synth.normal_bf16(gd, (B, chunk, 1, D), device="cuda")
        api.kv_append_fp8(kc, ks, None, None, kn, None,
                          torch.full((B,), p0, dtype=torch.int32, device="cuda"), g.kind)
    ctx_t = torch.from_numpy(ctx).cuda()
    q = synth.normal_bf16(gd, (B, g.num_q_heads, D), device="cuda")
    out = api.decode_fp8(q, kc, ks, None, None, ctx_t, ctx_t - 1, g.window, g.softcap,
                         g.q_scale, g.kind, max_ctx=C)
    torch.cuda.synchronize()
    rows = sorted({0, int(np.argmax(ctx)), int(np.argmin(ctx))})
    log(f"fp8 global rows {rows} ctx {ctx[rows].tolist()}")
    kcr, ksr = kc[rows].cpu().numpy(), ks[rows].cpu().numpy()
    ref, _, _, _ = oracle.decode_fp8_multi(synth.bits(q[rows].cpu())[:, None], kcr, ksr, None,
                                           None, ctx[rows], ctx[rows] - 1, g.window, g.softcap,
                                           g.q_scale, g.kind)
    assert_parity(out[rows].unsqueeze(1), ref, "fp8 global full size")


@pytest.mark.parametrize("D,G,Hkv,k_eq_v,T", [(256, 2, 4, False, 8), (128, 4, 2, False, 4),
                                              (512, 16, 1, True, 2), (256, 8, 1, True, 3)])
def test_fp8_multi_token_matrix_cores_match_vector_kernel_and_oracle(D, G, Hkv, k_eq_v, T):
    """Several query tokens over fp8 caches on the matrix cores (16 query rows per KV head,
    codes widened to bf16, K scales on the logits, V scales on the value weights, the
    work-group's waves merged in LDS) and on the vector kernel: both match the oracle,
    with one split per unit and with several (merge kernel), over ring windows at the
    wrap edges."""
    w = 64
    cap, window = w + T - 1, w
    ctx = [T, w - 1, w, w + 1, w + T - 1, 2 * w + 3, 5 * w - 1]
    inp = Fp8Inputs(777 + D + T, len(ctx), T, G * Hkv, Hkv, D, cap, k_eq_v, ctx)
    inp.poison(window, api.RING).to_device()
    ref, _ = inp.oracle(window, 30.0, default_scale(D), api.RING)
    for impl in [api.IMPL_MFMA, api.IMPL_VALU]:
        for split in [0, 64]:
            out = inp.run(window, 30.0, default_scale(D), api.RING, max_ctx=max(ctx), impl=impl,
                          split_keys=split)
            assert_parity(out, ref, f"fp8 T={T} D={D} G={G} impl={impl} split={split}")


def test_fp8_spec_decode_layer_full_size_sampled_rows():
    """The 12B sliding layer verifying 8 tokens (ring 1031, w 1024) over an fp8 cache
    filled by quantizing appends; sampled rows against the oracle (BF16 queries, FP8 KV,
    spec decode on a sliding window: the combination reported to corrupt in another
    engine)."""
    w = wl.FP8_SPEC_DECODE_SLIDING
    g = w.layers[0]
    B, T, Hkv, D, W = w.batch, w.tokens, g.num_kv_heads, g.head_dim, g.capacity
    ctx = synth.uniform_int(synth.generator(w.seed), B, w.ctx_lo, w.ctx_hi).numpy() \
        .astype(np.int32)
    gd = synth.generator(78, device="cuda")
    kc = torch.empty((B, Hkv, W, D), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    ks = torch.empty((B, Hkv, W), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    ctx_t = torch.from_numpy(ctx).cuda()
    for part in range(0, W, 512):
        n = min(512, W - part)
        kn = synth.normal_bf16(gd, (B, n, Hkv, D), device="cuda")
        vn = synth.normal_bf16(gd, (B, n, Hkv, D), device="cuda")
        api.kv_append_fp8(kc, ks, vc, vs, kn, vn, ctx_t - W + part, api.RING)
    q = synth.normal_bf16(gd, (B, T, g.num_q_heads, D), device="cuda")
    out = api.decode_fp8(q, kc, ks, vc, vs, ctx_t, ctx_t - T, g.window, g.softcap, g.q_scale,
                         g.kind, max_ctx=w.ctx_hi)
    torch.cuda.synchronize()
    rows = sorted({0, 1, int(np.argmax(ctx)), int(np.argmin(ctx))})
    log(f"fp8 spec decode rows {rows}")
    ref, _, _, flags = oracle.decode_fp8_multi(
        synth.bits(q[rows].cpu()), kc[rows].cpu().numpy(), ks[rows].cpu().numpy(),
        vc[rows].cpu().numpy(), vs[rows].cpu().numpy(), ctx[rows], ctx[rows] - T, g.window,
        g.softcap, g.q_scale, g.kind)
    assert not flags.any()
    assert_parity(out[rows], ref, "fp8 spec decode full size")
