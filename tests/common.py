"""Shared helpers for the GPU parity tests: seeded inputs, poisoning, oracle calls and
the tolerance gate.

Tolerance: max |gpu - oracle| <= 1e-2 and ||gpu - oracle||_2 / ||oracle||_2 <= 2e-3 over
the compared outputs of one call, with the oracle in fp64 on the same bf16 inputs.
"""
import math

import numpy as np
import torch

import oracle
from decode_attention_split_amd import synth

TOL_MAX_ABS = 1e-2
TOL_REL_L2 = 2e-3
BF16_NAN = synth.BF16_NAN


def log(msg):
    print(msg, flush=True)


class LayerInputs:
    """Host copies (uint16 bits / int32) and device tensors of one layer's decode call."""

    def __init__(self, q, k, v, ctx, qpos):
        self.q_bits, self.k_bits = q, k
        self.v_bits = v
        self.ctx = np.asarray(ctx, np.int32)
        self.qpos = np.asarray(qpos, np.int32)

    def to_device(self, device="cuda"):
        self.q = synth.from_bits(self.q_bits, device)
        self.k = synth.from_bits(self.k_bits, device)
        self.v = None if self.v_bits is None else synth.from_bits(self.v_bits, device)
        self.ctx_t = torch.from_numpy(self.ctx.copy()).to(device)
        self.qpos_t = torch.from_numpy(self.qpos.copy()).to(device)
        return self


def gen_layer(seed, B, Hq, Hkv, D, cap, k_eq_v, ctx_lo, ctx_hi, ctx=None):
    """Seeded draws in the order ctx_lens, q, K, V (every physical slot filled)."""
    gen = synth.generator(seed)
    c = synth.uniform_int(gen, B, ctx_lo, ctx_hi)
    if ctx is not None:
        c = torch.as_tensor(np.asarray(ctx, np.int32))
    q = synth.bits(synth.normal_bf16(gen, (B, Hq, D)))
    k = synth.bits(synth.normal_bf16(gen, (B, Hkv, cap, D)))
    v = None if k_eq_v else synth.bits(synth.normal_bf16(gen, (B, Hkv, cap, D)))
    ctx_np = c.numpy().astype(np.int32)
    return LayerInputs(q, k, v, ctx_np, ctx_np - 1)


def poison_invalid_slots(inp: LayerInputs, window, kind, cap):
    """Fill every slot outside each row's valid set (per the oracle) with bf16 NaN, so
    any stray read turns the GPU output NaN."""
    for b in range(inp.ctx.shape[0]):
        _, slots = oracle.valid_positions(inp.ctx[b], inp.qpos[b], window, kind, cap)
        keep = np.zeros(cap, bool)
        keep[slots] = True
        drop = np.flatnonzero(~keep)
        if drop.size == 0:
            continue
        for bits in [inp.k_bits] + ([inp.v_bits] if inp.v_bits is not None else []):
            if drop[-1] - drop[0] + 1 == drop.size:  # one run of slots: a plain slice
                bits[b][:, drop[0]:drop[-1] + 1, :] = BF16_NAN
            else:
                bits[b][:, drop, :] = BF16_NAN


def oracle_out(inp: LayerInputs, window, softcap, scale, kind, rows=None):
    """fp64 oracle output [B', Hq, D] for the selected batch rows (default all)."""
    if rows is None:
        rows = np.arange(inp.q_bits.shape[0])
    rows = np.asarray(rows)
    out, _, _, _ = oracle.decode(inp.q_bits[rows], inp.k_bits[rows],
                                 None if inp.v_bits is None else inp.v_bits[rows],
                                 inp.ctx[rows], inp.qpos[rows], window, softcap, scale, kind)
    return out


def errors(gpu, ref):
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else gpu
    d = g - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_parity(gpu, ref, what=""):
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else gpu
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    max_abs, rel = errors(g, ref)
    log(f"  parity {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= TOL_MAX_ABS, f"{what}: max_abs {max_abs}"
    assert rel <= TOL_REL_L2, f"{what}: rel_l2 {rel}"
    return max_abs, rel


def f32(x):
    return float(np.float32(x))


def default_scale(D):
    return f32(1.0 / math.sqrt(D))
