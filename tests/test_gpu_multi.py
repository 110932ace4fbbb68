"""GPU: multi-token decode (T query tokens per row, each masked at its own position), the
T-token append and the per-token precondition flags, against the fp64 oracle.

Parity cases poison every slot outside the union of a row's tokens' valid sets with bf16
NaN, so a stray read shows up as a NaN output.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_split_amd import api, synth

from common import BF16_NAN, assert_parity, default_scale, log

pytestmark = pytest.mark.gpu


class MultiInputs:
    def __init__(self, seed, B, T, Hq, Hkv, D, cap, k_eq_v, ctx, q0=None):
        gen = synth.generator(seed)
        self.q_bits = synth.bits(synth.normal_bf16(gen, (B, T, Hq, D)))
        self.k_bits = synth.bits(synth.normal_bf16(gen, (B, Hkv, cap, D)))
        self.v_bits = None if k_eq_v else synth.bits(synth.normal_bf16(gen, (B, Hkv, cap, D)))
        self.ctx = np.asarray(ctx, np.int32)
        self.q0 = self.ctx - T if q0 is None else np.asarray(q0, np.int32)
        self.T, self.cap = T, cap

    def poison(self, window, kind):
        for bits in [self.k_bits] + ([self.v_bits] if self.v_bits is not None else []):
            for b in range(bits.shape[0]):
                keep = np.zeros(self.cap, bool)
                for t in range(self.T):
                    _, slots = oracle.valid_positions(self.ctx[b], self.q0[b] + t, window, kind,
                                                      self.cap)
                    keep[slots] = True
                bits[b][:, ~keep, :] = BF16_NAN
        return self

    def to_device(self):
        self.q = synth.from_bits(self.q_bits, "cuda")
        self.k = synth.from_bits(self.k_bits, "cuda")
        self.v = None if self.v_bits is None else synth.from_bits(self.v_bits, "cuda")
        self.ctx_t = torch.from_numpy(self.ctx.copy()).cuda()
        self.q0_t = torch.from_numpy(self.q0.copy()).cuda()
        return self

    def oracle(self, window, softcap, scale, kind, rows=None):
        rows = np.arange(self.q_bits.shape[0]) if rows is None else np.asarray(rows)
        out, _, _, flags = oracle.decode_multi(
            self.q_bits[rows], self.k_bits[rows],
            None if self.v_bits is None else self.v_bits[rows], self.ctx[rows], self.q0[rows],
            window, softcap, scale, kind)
        return out, flags

    def run(self, window, softcap, scale, kind, **kw):
        out = api.decode_multi(self.q, self.k, self.v, self.ctx_t, self.q0_t, window, softcap,
                               scale, kind, **kw)
        torch.cuda.synchronize()
        return out


@pytest.mark.parametrize("D,G,Hkv", [(128, 2, 2), (256, 1, 2), (256, 2, 4), (256, 4, 1),
                                     (512, 8, 1), (512, 16, 1), (128, 16, 1)])
@pytest.mark.parametrize("T", [2, 5, 8])
@pytest.mark.parametrize("kind", [api.RING, api.LINEAR])
@pytest.mark.parametrize("impl", [api.IMPL_VALU, api.IMPL_MFMA], ids=["valu", "mfma"])
def test_multi_token_parity_sweep(D, G, Hkv, T, kind, impl):
    """Several splits, chunks of tokens and ragged tails; rows whose first tokens precede
    the sequence start (negative positions attend to nothing).  Both implementations: the
    vector kernel and the matrix-core kernel for 16 query rows per KV head."""
    if impl == api.IMPL_MFMA and D == 512 and G != 16:
        pytest.skip("matrix-core multi-token path: head_dim 512 only with K = V")
    w = 96
    if kind == api.RING:
        cap, window = w + T - 1, w
        ctx = [1, T, w, w + 1, 3 * cap + 5]
        max_ctx = max(ctx)
    else:
        cap, window = 400, (w if G % 2 == 0 else 0)
        ctx = [1, T, 150, 399, 400]
        max_ctx = cap
    k_eq_v = (G == 16)
    inp = MultiInputs(D * 10 + G * 100 + T, len(ctx), T, G * Hkv, Hkv, D, cap, k_eq_v, ctx)
    inp.poison(window, kind).to_device()
    softcap = 30.0 if T % 2 == 0 else 0.0
    ref, _ = inp.oracle(window, softcap, default_scale(D), kind)
    for split in [0, 64]:
        out = inp.run(window, softcap, default_scale(D), kind, max_ctx=max_ctx, split_keys=split,
                      impl=impl)
        assert_parity(out, ref, f"D={D} G={G} T={T} kind={kind} split={split} impl={impl}")


@pytest.mark.parametrize("W", [64, 1024])
def test_multi_token_window_edges(W):
    """Draft tokens straddling multiples of the window and of the ring: where a
    spec-decode kernel mis-selected sliding-window keys at certain seq_len alignments."""
    T = 8
    w = W
    cap = w + T - 1
    ctxs = [T, w - 1, w, w + 1, w + T - 1, 2 * w, 2 * w + 3, 3 * w + T, 5 * w - 1]
    inp = MultiInputs(W + 7, len(ctxs), T, 16, 8, 256, cap, False, ctxs)
    inp.poison(w, api.RING).to_device()
    ref, flags = inp.oracle(w, 50.0, 1.0 / 16, api.RING)
    assert not flags.any()
    for split in [0, 64, 256]:
        out = inp.run(w, 50.0, 1.0 / 16, api.RING, max_ctx=max(ctxs), split_keys=split)
        assert_parity(out, ref, f"W={W} split={split}")


def test_multi_token_causal_inside_the_cache():
    """Query tokens below the newest cached position (q_pos + T < ctx): each token still
    sees only positions up to its own."""
    T = 4
    ctx = [50, 300, 300]
    q0 = [10, 0, 250]
    inp = MultiInputs(17, 3, T, 8, 2, 256, 300, False, ctx, q0)
    inp.poison(0, api.LINEAR).to_device()
    ref, _ = inp.oracle(0, 0.0, 0.0625, api.LINEAR)
    out = inp.run(0, 0.0, 0.0625, api.LINEAR, max_ctx=300)
    assert_parity(out, ref, "causal inside")


def test_multi_T1_equals_single_token_decode_bitwise():
    inp = MultiInputs(21, 4, 1, 16, 8, 256, 128, False, [1, 64, 128, 200])
    inp.poison(128, api.RING).to_device()
    a = inp.run(128, 0.0, 0.0625, api.RING, max_ctx=200, deterministic=True)
    b = api.decode(inp.q[:, 0].contiguous(), inp.k, inp.v, inp.ctx_t, inp.q0_t, 128, 0.0, 0.0625,
                   api.RING, max_ctx=200, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], b)


def test_spec_decode_sliding_layer_full_size_sampled_rows():
    """The 12B sliding layer verifying 7 draft tokens (T = 8): B 64, ring of 1031 slots,
    window 1024, ctx U[512, 8192]."""
    T, w = 8, 1024
    gen = synth.generator(3)
    ctx = synth.uniform_int(gen, 64, 512, 8192).numpy().astype(np.int32)
    inp = MultiInputs(33, 64, T, 16, 8, 256, w + T - 1, False, ctx).to_device()
    out = inp.run(w, 50.0, 1.0 / 16, api.RING, max_ctx=8192)  # matrix cores (auto)
    rows = sorted({0, 1, int(np.argmax(ctx)), int(np.argmin(ctx))})
    ref, _ = inp.oracle(w, 50.0, 1.0 / 16, api.RING, rows=rows)
    log(f"spec decode rows {rows}")
    assert_parity(out[rows], ref, "spec decode T=8")
    # the vector kernel on the same inputs agrees on every row
    out_v = inp.run(w, 50.0, 1.0 / 16, api.RING, max_ctx=8192, impl=api.IMPL_VALU)
    assert_parity(out, out_v.double().cpu().numpy(), "spec decode mfma vs valu")


def test_append_multi_matches_oracle_bitwise():
    B, T, Hkv, D = 3, 6, 2, 256
    for kind, cap, pos0 in [(api.RING, 4, [0, 7, 1000]), (api.LINEAR, 16, [-2, 5, 12])]:
        gen = synth.generator(40 + kind)
        k = synth.normal_bf16(gen, (B, Hkv, cap, D))
        v = synth.normal_bf16(gen, (B, Hkv, cap, D))
        kn = synth.normal_bf16(gen, (B, T, Hkv, D))
        vn = synth.normal_bf16(gen, (B, T, Hkv, D))
        ref_k, ref_v = synth.bits(k).copy(), synth.bits(v).copy()
        if kind == api.RING:
            oracle.append_tokens(ref_k, synth.bits(kn), np.asarray(pos0, np.int32), kind)
            oracle.append_tokens(ref_v, synth.bits(vn), np.asarray(pos0, np.int32), kind)
        else:
            # the oracle refuses out-of-range positions; the library skips them, so the
            # expected cache is the definition: write token t at pos0 + t when 0 <= p < C
            for b in range(B):
                for t in range(T):
                    p = pos0[b] + t
                    if 0 <= p < cap:
                        ref_k[b, :, p] = synth.bits(kn)[b, t]
                        ref_v[b, :, p] = synth.bits(vn)[b, t]
        kd, vd = k.cuda(), v.cuda()
        api.kv_append_multi(kd, vd, kn.cuda(), vn.cuda(),
                            torch.tensor(pos0, dtype=torch.int32, device="cuda"), kind)
        torch.cuda.synchronize()
        assert np.array_equal(synth.bits(kd.cpu()), ref_k), kind
        assert np.array_equal(synth.bits(vd.cpu()), ref_v), kind


def test_validate_multi_matches_oracle_flags():
    T, w, W = 4, 8, 8  # a ring of exactly w slots: the first tokens need evicted keys
    ctx = np.array([5, 8, 30, 0], np.int32)
    q0 = ctx - T
    shape = api.make_shape(4, 2, 1, 128, W, api.RING, 30)
    # the host refuses this ring for decoding T tokens (window + T - 1 > W) ...
    with pytest.raises(api.GemmaAttnError) as e:
        api.validate_multi(shape, T, torch.from_numpy(ctx).cuda(), torch.from_numpy(q0).cuda(), w)
    assert e.value.code == -6
    # ... and accepts it while the context never exceeds W, flagging per token
    shape = api.make_shape(4, 2, 1, 128, W, api.RING, 8)
    ctx = np.array([5, 8, 8, 0], np.int32)
    q0 = np.array([1, 4, -1, 0], np.int32)
    flags = api.validate_multi(shape, T, torch.from_numpy(ctx).cuda(),
                               torch.from_numpy(q0).cuda(), w).cpu().numpy()
    q = np.zeros((4, T, 2, 128), np.uint16)
    kc = np.zeros((4, 1, W, 128), np.uint16)
    _, _, _, ref = oracle.decode_multi(q, kc, None, ctx, q0, w, 0.0, 1.0, oracle.RING)
    assert np.array_equal(flags & 15, ref), (flags, ref)


@pytest.mark.parametrize("D,G,Hkv,k_eq_v,split", [(256, 2, 8, False, 0), (256, 2, 8, False, 64),
                                                  (512, 16, 1, True, 0)])
def test_matrix_core_multi_token_repeats_bits(D, G, Hkv, k_eq_v, split):
    """The multi-token matrix-core kernel is deterministic without any option: its tiles
    go to the waves of a split in a fixed order and the waves (and splits) merge in a
    fixed order, so repeated calls give identical bits, with one split per unit and with
    several."""
    T = 16 // G if G < 16 else 2
    ctx = [T, 100, 900, 3000, 4096, 777, 64, 2500]
    inp = MultiInputs(4321 + D, len(ctx), T, G * Hkv, Hkv, D, 4096, k_eq_v, ctx).to_device()
    args = (0, 0.0, default_scale(D), api.LINEAR)
    first = inp.run(*args, impl=api.IMPL_MFMA, split_keys=split, max_ctx=4096)
    for _ in range(3):
        again = inp.run(*args, impl=api.IMPL_MFMA, split_keys=split, max_ctx=4096)
        assert torch.equal(first, again)
    ref, _ = inp.oracle(*args)
    assert_parity(first, ref, f"repeat D={D} split={split}")


# ------------------------------------------------------------------ chunked prefill sizes

def _prefill_ctxs(T, w):
    """Contexts around window and ring edges for a chunk of T tokens ending at ctx - 1."""
    return [T, w - 1, w, w + 1, w + T - 1, w + T, 2 * w + 3, 3 * w + T - 5]


@pytest.mark.parametrize("T", [64, 256])
@pytest.mark.parametrize("impl", [api.IMPL_AUTO, api.IMPL_VALU], ids=["auto", "valu"])
def test_chunked_prefill_sliding_12b_geometry(T, impl):
    """A prefill chunk of T = 64 / 256 tokens on the 12B sliding geometry (16 query heads
    on 8 KV heads, head_dim 256, window 1024, soft-cap 50) over a ring of w + T - 1 slots,
    contexts at window and ring edges; every never-valid slot poisoned with bf16 NaN.
    Element-wise against the oracle's multi-token definition."""
    w = 1024
    cap = w + T - 1
    ctx = _prefill_ctxs(T, w)
    inp = MultiInputs(5000 + T, len(ctx), T, 16, 8, 256, cap, False, ctx)
    inp.poison(w, api.RING).to_device()
    log(f"chunked prefill sliding T={T} impl={impl} ctx={ctx}")
    ref, flags = inp.oracle(w, 50.0, 1.0 / 16, api.RING)
    assert not flags.any()
    for split in ([0, 256] if impl == api.IMPL_AUTO else [0]):
        out = inp.run(w, 50.0, 1.0 / 16, api.RING, max_ctx=max(ctx), split_keys=split, impl=impl)
        assert_parity(out, ref, f"sliding T={T} impl={impl} split={split}")


@pytest.mark.parametrize("T", [64, 256])
def test_chunked_prefill_global_kv_shared_geometry(T):
    """A prefill chunk of T tokens on the K = V global geometry (16 query heads on one KV
    head, head_dim 512, linear cache, full causal): each token sees every position up to
    its own.  Positions past ctx - 1 are poisoned with bf16 NaN."""
    C = 4096
    ctx = [T, T + 1, 700, 1500] if T == 256 else [T, 1000, 2047, 3001]
    inp = MultiInputs(6000 + T, len(ctx), T, 16, 1, 512, C, True, ctx)
    inp.poison(0, api.LINEAR).to_device()
    log(f"chunked prefill global T={T} ctx={ctx}")
    scale = default_scale(512)
    ref, flags = inp.oracle(0, 0.0, scale, api.LINEAR)
    assert not flags.any()
    for split in [0, 512]:
        out = inp.run(0, 0.0, scale, api.LINEAR, max_ctx=C, split_keys=split)
        assert_parity(out, ref, f"global T={T} split={split}")


def _sampled_tokens_vs_oracle(inp, toks, window, softcap, scale, kind, out, what):
    """Tokens `toks` of every row against the oracle's single-token definition at their
    own positions (q_pos + t)."""
    for t in toks:
        ref, _, _, flags = oracle.decode_multi(
            inp.q_bits[:, t:t + 1], inp.k_bits, inp.v_bits, inp.ctx, inp.q0 + t, window,
            softcap, scale, kind)
        assert not flags.any()
        assert_parity(out[:, t:t + 1], ref, f"{what} token {t}")


def test_chunked_prefill_at_the_token_limit():
    """T = 4096 query tokens per row (the library's limit) on the 12B sliding geometry
    (ring of w + T - 1 = 5119 slots, one row starting at position 0 and one wrapped past the
    ring) and on the K = V global geometry (linear cache of 8192); every never-valid slot
    NaN-poisoned, the whole output finite, sampled tokens against the oracle."""
    T, w = 4096, 1024
    toks = [0, 1, w - 1, w, 2047, 3000, T - 2, T - 1]
    inp = MultiInputs(7100, 2, T, 16, 8, 256, w + T - 1, False, [T, 7000])
    inp.poison(w, api.RING).to_device()
    log("chunked prefill sliding T=4096")
    out = inp.run(w, 50.0, 1.0 / 16, api.RING, max_ctx=7000)
    assert torch.isfinite(out).all()
    _sampled_tokens_vs_oracle(inp, toks, w, 50.0, 1.0 / 16, api.RING, out, "sliding T=4096")
    del inp, out
    inp = MultiInputs(7200, 1, T, 16, 1, 512, 8192, True, [6000])
    inp.poison(0, api.LINEAR).to_device()
    log("chunked prefill global T=4096")
    scale = default_scale(512)
    out = inp.run(0, 0.0, scale, api.LINEAR, max_ctx=8192)
    assert torch.isfinite(out).all()
    _sampled_tokens_vs_oracle(inp, toks, 0, 0.0, scale, api.LINEAR, out, "global T=4096")
