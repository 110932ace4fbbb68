"""CPU pins of the oracle's rotary position embedding (RoPE) and its bf16 rounding.

Definition pinned here: with H = D/2, elements i and i + H form rotate-half pair i, which
turns by the angle p * base^(-2i/D) for i < R/2 (R the rotated width); every other element
passes through; the result is computed in double and rounded once to bf16 (nearest, ties
to even).  Sliding layers: base 10,000, R = D (the "default" rope type); full layers: base
1,000,000, R = D/4 (the "proportional" type with a partial rotary factor of 1/4).  Besides
closed forms and invariants, the oracle is compared with the transformers library's
Gemma 4 rotary embedding and its rotate-half application for both layer types.
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
    H = D // 2
    for i in [0, 1, R // 6, R // 2 - 1]:
        for p in [1, 37, 4095, 32767]:
            x = np.zeros((D,), np.uint16)
            x[i] = bf16_bits_of([1.0])[0]
            _, y = oracle.rope(x, [p], base, R)
            ang = p * base ** (-2.0 * i / D)
            assert y[i] == pytest.approx(math.cos(ang), abs=1e-14)
            assert y[i + H] == pytest.approx(math.sin(ang), abs=1e-14)
            others = np.delete(y, [i, i + H])
            assert (others == 0).all()


@pytest.mark.parametrize("D,R", [(512, 128), (256, 64)])
def test_pairs_past_the_rotated_width_pass_through(D, R):
    # a unit vector on a pair i >= R/2 (either half) stays where it is at any position
    H = D // 2
    for d in [R // 2, H - 1, H + R // 2, D - 1]:
        x = np.zeros((D,), np.uint16)
        x[d] = bf16_bits_of([1.0])[0]
        y16, y = oracle.rope(x, [12345], 1e6, R)
        assert y16[d] == x[d]
        assert (np.delete(y, [d]) == 0).all()  # (zero pairs that rotate may turn to -0)


def test_rotation_keeps_pair_norms_and_passes_the_rest_through():
    rng = np.random.default_rng(2)
    D, R = 512, 128
    H, n = D // 2, R // 2
    x = bf16_random(rng, (8, D))
    pos = rng.integers(0, 30000, 8)
    y16, y = oracle.rope(x, pos, 1e6, R)
    xf = brute.widen_bf16(x)
    n_in = xf[:, :n] ** 2 + xf[:, H:H + n] ** 2
    n_out = y[:, :n] ** 2 + y[:, H:H + n] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12, atol=1e-15)
    assert np.array_equal(y16[:, n:H], x[:, n:H])
    assert np.array_equal(y16[:, H + n:], x[:, H + n:])
    # the bits are the values rounded once
    assert np.array_equal(y16, np.vectorize(oracle.f64_to_bf16)(y).astype(np.uint16))


@pytest.mark.parametrize("layer_type", ["sliding_attention", "full_attention"])
def test_matches_the_library_gemma4_rotary_embedding(layer_type):
    """The transformers library's Gemma 4 model code: its rotary embedding module (the
    "default" rope type on sliding layers, "proportional" with partial rotary factor 1/4
    on full layers, from the model config's defaults) and its rotate-half application.
    Its angles are float32 products (inverse frequency x position), so values agree to
    the float32 angle error; elements it leaves alone must come back bit for bit."""
    pytest.importorskip("transformers")
    from transformers.models.gemma4 import configuration_gemma4 as cg
    from transformers.models.gemma4 import modeling_gemma4 as mg
    cfg = cg.Gemma4TextConfig(num_hidden_layers=6, hidden_size=64, num_attention_heads=2,
                              intermediate_size=128, vocab_size=128, head_dim=256,
                              global_head_dim=512)
    emb = mg.Gemma4TextRotaryEmbedding(cfg)
    D = 512 if layer_type == "full_attention" else 256
    base = cfg.rope_parameters[layer_type]["rope_theta"]
    inv_freq = getattr(emb, f"{layer_type}_inv_freq")
    R = 2 * int(torch.count_nonzero(inv_freq))
    assert inv_freq.numel() == D // 2
    assert (base, R) == ((1e6, D // 4) if layer_type == "full_attention" else (1e4, D))
    rng = np.random.default_rng(11)
    pos = np.array([0, 1, 37, 1000, 4000], np.int64)
    x = bf16_random(rng, (len(pos), D))
    y16, y = oracle.rope(x, pos, base, R)
    xf = torch.from_numpy(brute.widen_bf16(x))
    cos, sin = emb(xf[None, :, None, :], torch.from_numpy(pos)[None, :], layer_type)
    ref = mg.apply_rotary_pos_emb(xf[None, :, None, :], cos, sin, unsqueeze_dim=2)[0, :, 0, :]
    ref = ref.numpy()
    assert np.abs(y - ref).max() < 4e-3  # |x| <~ 4, angles within ~6e-8 * 4000 rad
    moved = np.abs(ref - brute.widen_bf16(x)) > 0
    assert np.array_equal(np.abs(y - brute.widen_bf16(x)) > 0, moved)


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
