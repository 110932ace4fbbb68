"""CPU pins of the oracle's rotary position embedding (RoPE) and its bf16 rounding.

Reading pinned here: the first R elements of a head rotate in rotate-half pairs
(i, i + R/2) by the angle p * base^(-2i/R); the rest pass through; the result is computed
in double and rounded once to bf16 (nearest, ties to even).  Bases: 10,000 (sliding
layers, whole head) and 1,000,000 (full layers, partial rotary on the low part).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute


def bf16_bits_of(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_f64_to_bf16_rounds_directly_to_nearest_even():
    rng = np.random.default_rng(0)
    xs = rng.standard_normal(2000).astype(np.float32) * 10.0 ** rng.integers(-5, 5, 2000)
    got = np.array([oracle.f64_to_bf16(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, bf16_bits_of(xs))  # float32 inputs: torch's RNE
    # a value just above a bf16 tie whose float32 rounding lands exactly on the tie: a
    # float step would round it down to 1.0, direct rounding goes up to 1 + 2^-7
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.f64_to_bf16(x) == int(bf16_bits_of([1.0 + 2.0 ** -7])[0])
    assert oracle.f64_to_bf16(-x) == int(bf16_bits_of([-(1.0 + 2.0 ** -7)])[0])
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == int(bf16_bits_of([1.0])[0])  # a true tie


def bf16_random(rng, shape):
    return bf16_bits_of(rng.standard_normal(shape))


@pytest.mark.parametrize("D,R,base", [(256, 256, 1e4), (512, 128, 1e6), (128, 64, 1e4)])
def test_identity_at_position_zero_and_without_rotary(D, R, base):
    x = bf16_random(np.random.default_rng(1), (3, D))
    y, _ = oracle.rope(x, [0, 0, 0], base, R)
    assert np.array_equal(y, x)
    y, _ = oracle.rope(x, [5, 100, 7000], base, 0)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("D,R,base", [(256, 256, 1e4), (512, 128, 1e6), (512, 512, 1e6)])
def test_unit_vectors_rotate_by_the_closed_form_angle(D, R, base):
    half = R // 2
    for i in [0, 1, half // 3, half - 1]:
        for p in [1, 37, 4095, 32767]:
            x = np.zeros((D,), np.uint16)
            x[i] = bf16_bits_of([1.0])[0]
            _, y = oracle.rope(x, [p], base, R)
            ang = p * base ** (-2.0 * i / R)
            assert y[i] == pytest.approx(math.cos(ang), abs=1e-14)
            assert y[i + half] == pytest.approx(math.sin(ang), abs=1e-14)
            others = np.delete(y, [i, i + half])
            assert (others == 0).all()


def test_rotation_keeps_pair_norms_and_passes_the_rest_through():
    rng = np.random.default_rng(2)
    D, R = 512, 128
    x = bf16_random(rng, (8, D))
    pos = rng.integers(0, 30000, 8)
    y16, y = oracle.rope(x, pos, 1e6, R)
    xf = brute.widen_bf16(x)
    h = R // 2
    n_in = xf[:, :h] ** 2 + xf[:, h:R] ** 2
    n_out = y[:, :h] ** 2 + y[:, h:R] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12, atol=1e-15)
    assert np.array_equal(y16[:, R:], x[:, R:])
    # the bits are the values rounded once
    assert np.array_equal(y16, np.vectorize(oracle.f64_to_bf16)(y).astype(np.uint16))


def test_scores_depend_only_on_the_position_difference():
    rng = np.random.default_rng(3)
    D, R = 256, 256
    q = bf16_random(rng, (D,))
    k = bf16_random(rng, (D,))
    scores = []
    for shift in [0, 100, 5000]:
        _, qr = oracle.rope(q, [900 + shift], 1e4, R)
        _, kr = oracle.rope(k, [870 + shift], 1e4, R)
        scores.append(float(np.dot(qr, kr)))
    np.testing.assert_allclose(scores, scores[0], rtol=1e-9)
