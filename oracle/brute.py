"""Dense numpy brute force for decode attention, tiny shapes only.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  A second, independent
formulation of the same definition that oracle.c implements: instead of visiting
valid positions one at a time it builds, per batch row, the full logits matrix
over every stored position 0..ctx-1 for all query heads at once, masks it with an
explicit -inf boolean mask, and applies a dense numpy softmax.  Shares no code
with oracle.c; bf16 widening is done here with numpy bit operations.

Readings (same as the oracle): window w > 0 keeps exactly the w positions
q_pos-w+1..q_pos; w <= 0 is full causal; soft-cap c*tanh(s/c) when 0 < c < inf;
query head h reads KV head h // (Hq/Hkv); empty row -> output 0, lse -inf.
"""
import numpy as np

LINEAR = 0
RING = 1


def widen_bf16(bits):
    """uint16 bf16 bit patterns -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def brute_decode(q, k_cache, v_cache, ctx_lens, q_pos, window, softcap, scale, kind):
    """Returns (out [B,Hq,D], lse [B,Hq]) in float64."""
    qf = widen_bf16(q)
    kf = widen_bf16(k_cache)
    vf = kf if v_cache is None else widen_bf16(v_cache)
    B, Hq, D = qf.shape
    _, Hkv, cap, _ = kf.shape
    G = Hq // Hkv
    scale = float(np.float32(scale))
    c = float(np.float32(softcap))
    cap_on = np.isfinite(c) and c > 0
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        ctx, qp = int(ctx_lens[b]), int(q_pos[b])
        if ctx <= 0:
            continue
        p = np.arange(ctx)
        mask = (p <= qp)
        if window > 0:
            mask &= p >= qp - window + 1
        if kind == RING:
            mask &= p >= ctx - cap
            storage = np.mod(p, cap)
        else:
            mask &= p < cap
            storage = np.minimum(p, cap - 1)  # masked-out rows read a harmless index
        # per-position K/V with KV heads expanded to query heads: [Hq, ctx, D]
        Kp = np.repeat(kf[b][:, storage, :], G, axis=0)
        Vp = np.repeat(vf[b][:, storage, :], G, axis=0)
        logits = scale * np.einsum("hd,hpd->hp", qf[b], Kp)
        if cap_on:
            logits = c * np.tanh(logits / c)
        logits = np.where(mask[None, :], logits, -np.inf)
        if not mask.any():
            continue
        mx = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - mx)
        ssum = e.sum(axis=1, keepdims=True)
        out[b] = np.einsum("hp,hpd->hd", e / ssum, Vp)
        lse[b] = mx[:, 0] + np.log(ssum[:, 0])
    return out, lse
