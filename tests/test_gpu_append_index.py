"""GPU: cache append and key-range selection must be bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_split_amd import api, synth

from common import log

pytestmark = pytest.mark.gpu

SENTINEL = 0x1234


@pytest.mark.parametrize("kind,cap,k_eq_v,D", [
    (api.RING, 32, False, 256),
    (api.RING, 7, False, 512),
    (api.LINEAR, 300, True, 512),
    (api.LINEAR, 100, False, 256),
])
def test_append_bit_exact(kind, cap, k_eq_v, D):
    log(f"append kind={kind} cap={cap} k_eq_v={k_eq_v} D={D}")
    rng = np.random.default_rng(cap + D)
    B, Hkv = 3, 2
    kc = np.full((B, Hkv, cap, D), SENTINEL, np.uint16)
    vc = None if k_eq_v else kc.copy()
    kc_d = synth.from_bits(kc, "cuda")
    vc_d = None if k_eq_v else synth.from_bits(vc, "cuda")
    offsets = np.array([0, 5, 11], np.int32)
    steps = 3 * cap + 4 if kind == api.RING else cap - 12
    for t in range(steps):
        pos = (t + offsets).astype(np.int32)
        kn = rng.integers(0, 1 << 16, size=(B, Hkv, D), dtype=np.uint16)
        vn = None if k_eq_v else rng.integers(0, 1 << 16, size=(B, Hkv, D), dtype=np.uint16)
        oracle.append(kc, kn, pos, kind)
        if not k_eq_v:
            oracle.append(vc, vn, pos, kind)
        api.kv_append(kc_d, vc_d, synth.from_bits(kn, "cuda"),
                      None if k_eq_v else synth.from_bits(vn, "cuda"),
                      torch.from_numpy(pos).cuda(), kind)
        if t % 17 == 0 or t == steps - 1:
            torch.cuda.synchronize()
            assert np.array_equal(synth.bits(kc_d), kc), f"K cache differs after step {t}"
            if not k_eq_v:
                assert np.array_equal(synth.bits(vc_d), vc), f"V cache differs after step {t}"
    if kind == api.LINEAR:  # untouched positions keep the sentinel
        assert (kc[0, :, steps:] == SENTINEL).all()


def test_append_skips_rows_with_out_of_range_positions():
    B, Hkv, D, cap = 3, 1, 256, 16
    kc = synth.from_bits(np.full((B, Hkv, cap, D), SENTINEL, np.uint16), "cuda")
    kn = synth.from_bits(np.full((B, Hkv, D), 0x3F80, np.uint16), "cuda")
    pos = torch.tensor([-1, 16, 3], dtype=torch.int32, device="cuda")
    api.kv_append(kc, None, kn, None, pos, api.LINEAR)
    got = synth.bits(kc)
    assert (got[0] == SENTINEL).all() and (got[1] == SENTINEL).all()
    assert (got[2, :, 3] == 0x3F80).all()
    assert (np.delete(got[2], 3, axis=1) == SENTINEL).all()


def range_cases():
    cases = []
    for W in [32, 64, 1024]:
        for w in [1, 2, W // 2, W - 1, W]:
            for ctx in [0, 1, w - 1, w, w + 1, 2 * w - 1, 2 * w, 2 * w + 1, W - 1, W, W + 1,
                        3 * W + 7, 8192]:
                for dq in [0, 1, 5]:
                    cases.append((api.RING, W, w, max(ctx, 0), max(ctx - 1 - dq, 0)))
    for C in [64, 4096]:
        for w in [0, 1, 33, C]:
            for ctx in [0, 1, 2, 63, 64, C - 1, C]:
                for dq in [0, 3]:
                    cases.append((api.LINEAR, C, w, ctx, max(ctx - 1 - dq, 0)))
    return cases


def test_key_ranges_match_the_oracle_exactly():
    """The (lo, hi, slot(lo), n) each decode kernel uses equals the oracle's valid set:
    a contiguous run of positions whose slots are slot(lo) + i wrapped at W."""
    cases = range_cases()
    groups = {}
    for kind, cap, w, ctx, qp in cases:
        groups.setdefault((kind, cap, w), []).append((ctx, qp))
    checked = 0
    for (kind, cap, w), rows in groups.items():
        ctx = torch.tensor([r[0] for r in rows], dtype=torch.int32, device="cuda")
        qp = torch.tensor([r[1] for r in rows], dtype=torch.int32, device="cuda")
        max_ctx = max(r[0] for r in rows)
        if kind == api.LINEAR or w <= 0:
            max_ctx = min(max_ctx, cap)
        s = api.make_shape(len(rows), 2, 1, 256, cap, kind, max_ctx)
        got = api.debug_ranges(s, ctx, qp, w).cpu().numpy()
        for i, (c, q) in enumerate(rows):
            pos, slots = oracle.valid_positions(c, q, w, kind, cap)
            lo, hi, slot_lo, n = got[i].tolist()
            assert n == len(pos), (kind, cap, w, c, q, got[i])
            if n:
                assert (lo, hi) == (pos[0], pos[-1])
                assert list(range(lo, hi + 1)) == pos.tolist()
                gpu_slots = [(slot_lo + j) % cap if kind == api.RING else slot_lo + j
                             for j in range(n)]
                assert gpu_slots == slots.tolist()
            checked += 1
    log(f"  {checked} rows checked")


def test_validate_flags_match_the_oracle():
    rows = [(70, 69, 32, api.RING, 32), (70, 69, 0, api.RING, 32), (32, 31, 0, api.RING, 32),
            (5, 5, 0, api.LINEAR, 8), (9, 8, 0, api.LINEAR, 8), (0, 0, 0, api.LINEAR, 8),
            (-1, 0, 0, api.LINEAR, 8), (40, 35, 4, api.RING, 8), (40, 2, 4, api.RING, 8)]
    for ctx, qp, w, kind, cap in rows:
        s = api.make_shape(1, 1, 1, 256, cap, kind, cap if (kind == api.LINEAR or w <= 0) else 64)
        f = api.validate(s, torch.tensor([ctx], dtype=torch.int32, device="cuda"),
                         torch.tensor([qp], dtype=torch.int32, device="cuda"), w)
        got = int(f.cpu()[0])
        assert got & 15 == oracle.row_flags(ctx, qp, w, kind, cap), (ctx, qp, w, kind, cap, got)
        assert bool(got & api.FLAG_OVER_MAX_CTX) == (ctx > s.max_ctx)
