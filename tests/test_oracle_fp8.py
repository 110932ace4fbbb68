"""CPU pins of the oracle's fp8 (e4m3) cache: code conversions, row quantization and
decode over quantized caches.

e4m3 here is the OCP 8-bit float with 4 exponent bits (bias 7), 3 mantissa bits, no
infinities and NaN at 0x7f / 0xff (torch.float8_e4m3fn is the same format and serves as
the library routine the conversions are checked against).  The fp8 decode is pinned to
the bf16 decode, which the other oracle tests pin: with power-of-two row scales every
cached value is exactly a bf16 value, so the two must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def e4m3_values_torch(codes):
    return torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_decode_matches_torch_and_the_format_definition():
    ref = e4m3_values_torch(range(256))
    for c in range(256):
        v = oracle.e4m3_to_f64(c)
        if c in (0x7F, 0xFF):
            assert np.isnan(v) and np.isnan(ref[c])
        else:
            assert v == ref[c], hex(c)
    # spot values of the format: smallest subnormal, smallest normal, one, largest
    assert oracle.e4m3_to_f64(0x01) == 2.0 ** -9
    assert oracle.e4m3_to_f64(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_f64(0x38) == 1.0
    assert oracle.e4m3_to_f64(0x7E) == 448.0
    assert oracle.e4m3_to_f64(0xB8) == -1.0


def test_encode_round_trips_and_rounds_to_nearest_even_like_torch():
    vals = np.array([oracle.e4m3_to_f64(c) for c in FINITE], np.float32)
    for c, v in zip(FINITE, vals):
        if v == 0:
            continue
        assert oracle.f32_to_e4m3(v) == c, hex(c)
    # midpoints between neighbours (ties) and points just off them
    pos = np.sort(np.unique(np.abs(vals)))
    xs = []
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((np.float64(a) + np.float64(b)) / 2)
        xs += [mid, np.nextafter(mid, np.float32(1e9)), np.nextafter(mid, np.float32(-1e9))]
    xs = np.array(xs + [-x for x in xs], np.float32)
    ref = torch.tensor(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f32_to_e4m3(x) for x in xs], np.uint8)
    assert np.array_equal(got, ref)
    assert oracle.f32_to_e4m3(-(2.0 ** -10)) == 0x80  # a negative tie to zero keeps its sign
    assert oracle.f32_to_e4m3(1e6) == 0x7E and oracle.f32_to_e4m3(-1e6) == 0xFE


def bf16_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def test_quantize_row_invariants():
    rng = np.random.default_rng(1)
    x = bf16_bits(rng.standard_normal((6, 256)).astype(np.float32) * np.array(
        [1, 1e-3, 50, 1e-6, 3, 1], np.float32)[:, None])
    x[5] = 0  # an all-zero row
    codes, scales = oracle.quantize_rows_fp8(x)
    xf = brute.widen_bf16(x)
    for r in range(5):
        amax = np.float32(np.abs(xf[r]).max())
        assert scales[r] == np.float32(amax / np.float32(448))
        i = int(np.argmax(np.abs(xf[r])))
        assert codes[r, i] in (0x7E, 0xFE)  # the largest magnitude maps to +-448
        deq = np.array([oracle.e4m3_to_f64(c) for c in codes[r]]) * float(scales[r])
        err = np.abs(deq - xf[r])
        # 3 mantissa bits: half an ulp is 2^-4 of the value (2^-10 * scale absolute in the
        # subnormal range), plus the float32 product x * (448 / amax)
        assert (err <= np.abs(xf[r]) * 2.0 ** -4 * (1 + 1e-6) + 2.0 ** -10 * scales[r]).all()
    assert (codes[5] == 0).all() and scales[5] == 0


def random_codes(rng, shape):
    return rng.choice(np.array(FINITE, np.uint8), size=shape)


def code_bits_as_bf16(codes):
    """bf16 bit patterns of the e4m3 values (every e4m3 value is a bf16 value)."""
    return bf16_bits(e4m3_values_torch(codes.reshape(-1)).reshape(codes.shape))


@pytest.mark.parametrize("k_eq_v", [False, True])
@pytest.mark.parametrize("kind,window,T", [(oracle.RING, 24, 1), (oracle.LINEAR, 0, 3),
                                           (oracle.RING, 20, 4)])
def test_fp8_decode_equals_bf16_decode_of_the_same_values(k_eq_v, kind, window, T):
    rng = np.random.default_rng(7 + T)
    B, Hq, Hkv, D, cap = 3, 4, 2, 64, 32
    kc = random_codes(rng, (B, Hkv, cap, D))
    vc = None if k_eq_v else random_codes(rng, (B, Hkv, cap, D))
    # power-of-two row scales: code * scale is still exactly a bf16 value
    ks = np.ldexp(1.0, rng.integers(-3, 4, (B, Hkv, cap))).astype(np.float32)
    vs = None if k_eq_v else np.ldexp(1.0, rng.integers(-3, 4, (B, Hkv, cap))).astype(np.float32)
    kb = bf16_bits(e4m3_values_torch(kc.reshape(-1)).reshape(kc.shape) * ks[..., None])
    vb = None if k_eq_v else bf16_bits(
        e4m3_values_torch(vc.reshape(-1)).reshape(vc.shape) * vs[..., None])
    q = bf16_bits(rng.standard_normal((B, T, Hq, D)).astype(np.float32))
    ctx = np.array([1, 17, 90], np.int32)
    q0 = ctx - T
    a = oracle.decode_fp8_multi(q, kc, ks, vc, vs, ctx, q0, window, 20.0, 0.2, kind)
    b = oracle.decode_multi(q, kb, vb, ctx, q0, window, 20.0, 0.2, kind)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[3], b[3])


def test_fp8_single_token_form():
    rng = np.random.default_rng(3)
    kc = random_codes(rng, (2, 1, 16, 32))
    ks = np.ones((2, 1, 16), np.float32)
    q = bf16_bits(rng.standard_normal((2, 4, 32)).astype(np.float32))
    ctx = np.array([5, 16], np.int32)
    a = oracle.decode_fp8_multi(q, kc, ks, None, None, ctx, ctx - 1, 0, 0.0, 0.3, oracle.LINEAR)
    b = oracle.decode(q, code_bits_as_bf16(kc), None, ctx, ctx - 1, 0, 0.0, 0.3, oracle.LINEAR)
    assert np.array_equal(a[0], b[0])


def test_append_fp8_quantizes_each_token_and_keeps_the_newest_per_slot():
    rng = np.random.default_rng(11)
    B, T, Hkv, D, W = 2, 6, 2, 32, 4
    codes = np.zeros((B, Hkv, W, D), np.uint8)
    scales = np.zeros((B, Hkv, W), np.float32)
    new = bf16_bits(rng.standard_normal((B, T, Hkv, D)).astype(np.float32))
    pos0 = np.array([0, 9], np.int32)
    oracle.append_fp8(codes, scales, new, pos0, oracle.RING)
    qc, qs = oracle.quantize_rows_fp8(new)
    for b in range(B):
        for s in range(W):
            t = max(t for t in range(T) if (pos0[b] + t) % W == s)
            assert np.array_equal(codes[b, :, s], qc[b, t]) and np.array_equal(scales[b, :, s],
                                                                              qs[b, t])
    # linear: out-of-range positions are skipped
    codes = np.zeros((1, 1, 8, D), np.uint8)
    scales = np.zeros((1, 1, 8), np.float32)
    oracle.append_fp8(codes, scales, new[:1, :, :1], np.array([-2], np.int32), oracle.LINEAR)
    qc, qs = oracle.quantize_rows_fp8(new[:1, :, :1])
    assert np.array_equal(codes[0, 0, :4], qc[0, 2:, 0]) and (codes[0, 0, 4:] == 0).all()
