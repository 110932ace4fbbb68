"""CPU pins of the oracle's multi-token decode (T consecutive query tokens per row).

Token t of row b sits at position q_pos0[b] + t and is masked at that position: causal
limit min(q_pos0 + t, ctx - 1), window q_pos0 + t - w + 1 .. q_pos0 + t, ring eviction
ctx - W.  Pinned against the dense numpy brute force (an independent formulation), the
single-token oracle on each token's causal prefix, a closed form (scale 0: mean of the
token's own window), and the ring sizing rule of speculative verification.
"""
import numpy as np
import pytest

import oracle
from oracle import brute


def bf16_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    u = x.view(np.uint32)
    # round to nearest even on the upper 16 bits
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def make(rng, B, T, Hq, Hkv, D, cap, k_eq_v):
    q = bf16_bits(rng, (B, T, Hq, D))
    k = bf16_bits(rng, (B, Hkv, cap, D))
    v = None if k_eq_v else bf16_bits(rng, (B, Hkv, cap, D))
    return q, k, v


@pytest.mark.parametrize("T", [1, 3, 8])
@pytest.mark.parametrize("kind,cap,window", [(oracle.LINEAR, 40, 0), (oracle.LINEAR, 40, 6),
                                             (oracle.RING, 16, 9)])
@pytest.mark.parametrize("G,Hkv,D", [(1, 2, 8), (2, 2, 8), (4, 1, 16), (16, 1, 8)])
def test_multi_matches_dense_brute_force_per_token(T, kind, cap, window, G, Hkv, D):
    rng = np.random.default_rng(T * 1000 + cap * 10 + G)
    B = 4
    q, k, v = make(rng, B, T, G * Hkv, Hkv, D, cap, k_eq_v=(G == 16))
    if kind == oracle.RING:
        ctx = np.array([1, T, 12, 30], np.int32)  # ring W = 16 >= w + T - 1 for T <= 8
    else:
        ctx = np.array([1, T, 17, cap], np.int32)
    q0 = ctx - T  # the usual layout: the T newest positions are the query tokens
    out, lse, _, flags = oracle.decode_multi(q, k, v, ctx, q0, window, 30.0, 0.3, kind)
    for t in range(T):
        ref, ref_lse = brute.brute_decode(q[:, t], k, v, ctx, q0 + t, window, 30.0, 0.3, kind)
        np.testing.assert_allclose(out[:, t], ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[:, t], ref_lse, rtol=1e-11, atol=1e-12)
    # a negative position (token before the sequence start) is flagged and attends to
    # nothing
    assert (flags[0, :T - 1] & oracle.FLAG_NEGATIVE).all() if T > 1 else True


def test_multi_T1_is_single_token_decode():
    rng = np.random.default_rng(7)
    q, k, v = make(rng, 3, 1, 8, 2, 64, 50, False)
    ctx = np.array([5, 50, 31], np.int32)
    a = oracle.decode_multi(q, k, v, ctx, ctx - 1, 20, 0.0, 0.125, oracle.LINEAR)
    b = oracle.decode(q[:, 0], k, v, ctx, ctx - 1, 20, 0.0, 0.125, oracle.LINEAR)
    assert np.array_equal(a[0][:, 0], b[0]) and np.array_equal(a[1][:, 0], b[1])
    assert np.array_equal(a[3][:, 0], b[3])


@pytest.mark.parametrize("window", [0, 7])
def test_each_token_equals_single_decode_on_its_causal_prefix(window):
    """Token t sees exactly what a single-token decode sees with the cache cut at its
    own position: same positions, same order, so the same bits."""
    rng = np.random.default_rng(11 + window)
    T = 5
    q, k, v = make(rng, 2, T, 4, 2, 32, 64, False)
    ctx = np.array([20, 64], np.int32)
    q0 = ctx - T
    out, lse, _, _ = oracle.decode_multi(q, k, v, ctx, q0, window, 0.0, 0.2, oracle.LINEAR)
    for t in range(T):
        o, l, _, _ = oracle.decode(q[:, t], k, v, q0 + t + 1, q0 + t, window, 0.0, 0.2,
                                   oracle.LINEAR)
        assert np.array_equal(out[:, t], o) and np.array_equal(lse[:, t], l)


def test_scale_zero_gives_mean_of_each_tokens_own_window():
    rng = np.random.default_rng(3)
    T, w, D, cap = 4, 5, 16, 30
    q, k, v = make(rng, 1, T, 2, 1, D, cap, False)
    ctx = np.array([cap], np.int32)
    q0 = ctx - T
    out, _, _, _ = oracle.decode_multi(q, k, v, ctx, q0, w, 0.0, 0.0, oracle.LINEAR)
    vf = brute.widen_bf16(v)[0, 0]
    for t in range(T):
        p_hi = int(q0[0]) + t
        expect = vf[p_hi - w + 1:p_hi + 1].mean(axis=0)
        for h in range(2):
            np.testing.assert_allclose(out[0, t, h], expect, rtol=1e-13, atol=1e-15)


def test_ring_of_w_plus_T_minus_1_slots_equals_linear_and_w_slots_evicts():
    """Verifying T draft tokens against a sliding window of w needs the ring to keep the
    w + T - 1 newest positions: token 0's window starts T - 1 positions before token
    T-1's.  With exactly w slots the first T - 1 tokens would need evicted keys, which
    the precondition flags report (the window-edge failure of spec decode on SWA)."""
    rng = np.random.default_rng(5)
    B, T, w, D, total = 2, 4, 8, 16, 40
    Hq, Hkv = 2, 1
    hist_k = bf16_bits(rng, (B, Hkv, total, D))
    hist_v = bf16_bits(rng, (B, Hkv, total, D))
    q = bf16_bits(rng, (B, T, Hq, D))
    ctx = np.array([total, 25], np.int32)
    q0 = ctx - T
    lin = oracle.decode_multi(q, hist_k, hist_v, ctx, q0, w, 0.0, 0.25, oracle.LINEAR)
    for W, ok in [(w + T - 1, True), (w, False)]:
        ring_k = np.zeros((B, Hkv, W, D), np.uint16)
        ring_v = np.zeros_like(ring_k)
        for b in range(B):
            for p in range(ctx[b]):
                ring_k[b, :, p % W] = hist_k[b, :, p]
                ring_v[b, :, p % W] = hist_v[b, :, p]
        out, lse, _, flags = oracle.decode_multi(q, ring_k, ring_v, ctx, q0, w, 0.0, 0.25,
                                                 oracle.RING)
        if ok:
            assert np.array_equal(out, lin[0]) and not flags.any()
        else:
            assert (flags[:, :T - 1] & oracle.FLAG_EVICTED).all()
            assert not flags[:, T - 1].any()
            assert np.array_equal(out[:, T - 1], lin[0][:, T - 1])


def test_append_tokens_keeps_the_newest_token_of_each_slot():
    rng = np.random.default_rng(9)
    B, T, Hkv, D, W = 2, 6, 1, 8, 4
    cache = np.zeros((B, Hkv, W, D), np.uint16)
    new = bf16_bits(rng, (B, T, Hkv, D))
    pos0 = np.array([0, 7], np.int32)
    oracle.append_tokens(cache, new, pos0, oracle.RING)
    for b in range(B):
        for s in range(W):
            ts = [t for t in range(T) if (pos0[b] + t) % W == s]
            assert np.array_equal(cache[b, :, s], new[b, max(ts)])
