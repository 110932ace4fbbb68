"""GPU: the allocation-free decode entry point (gemma_attn_decode_noalloc, through the C
ABI) against gemma_attn_decode_ex with a caller workspace, on the same inputs: two calls
in a row on each path, the second with a smaller input, bit for bit with the
deterministic option and within the parity bar without it; a call whose workspace would
exceed the fixed scratch is refused."""
import numpy as np
import pytest
import torch

from decode_attention_split_amd import api

from common import assert_parity, default_scale, gen_layer, log, oracle_out

pytestmark = pytest.mark.gpu


def _both(inp, window, softcap, scale, kind, max_ctx, **kw):
    ref = api.decode(inp.q, inp.k, inp.v, inp.ctx_t, inp.qpos_t, window, softcap, scale, kind,
                     max_ctx=max_ctx, **kw)
    got = api.decode_noalloc(inp.q, inp.k, inp.v, inp.ctx_t, inp.qpos_t, window, softcap,
                             scale, kind, max_ctx=max_ctx, **kw)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("case", ["global_mfma", "sliding_splits"])
def test_noalloc_equals_the_workspace_entry_point_on_two_calls(case):
    if case == "global_mfma":  # 16 query heads on one K = V head: partials + plan in scratch
        geo = dict(Hq=16, Hkv=1, D=512, k_eq_v=True, kind=api.LINEAR, window=0, softcap=0.0)
        sizes = [(12, 3000, 1, 3000), (5, 700, 1, 700)]  # (B, cap, ctx_lo, ctx_hi)
    else:  # the vector kernel with several splits per row: split partials in scratch
        geo = dict(Hq=8, Hkv=2, D=256, k_eq_v=False, kind=api.RING, window=512, softcap=30.0)
        sizes = [(6, 512, 300, 4000), (3, 512, 1, 900)]
    scale = default_scale(geo["D"])
    for i, (B, cap, lo, hi) in enumerate(sizes):
        inp = gen_layer(700 + i, B, geo["Hq"], geo["Hkv"], geo["D"], cap, geo["k_eq_v"], lo, hi)
        inp.to_device()
        max_ctx = cap if geo["kind"] == api.LINEAR else hi
        split = 128 if case == "sliding_splits" else 0
        log(f"noalloc {case} call {i}: B={B} cap={cap} ctx={inp.ctx.tolist()}")
        got, ref = _both(inp, geo["window"], geo["softcap"], scale, geo["kind"], max_ctx,
                         split_keys=split, deterministic=True)
        assert torch.equal(got, ref), (got - ref).abs().max().item()
        got, ref = _both(inp, geo["window"], geo["softcap"], scale, geo["kind"], max_ctx,
                         split_keys=split)
        assert_parity(got, ref.double().cpu().numpy(), f"noalloc vs workspace {case} call {i}")
        assert_parity(got, oracle_out(inp, geo["window"], geo["softcap"], scale, geo["kind"]),
                      f"noalloc vs oracle {case} call {i}")


def test_noalloc_refuses_a_call_beyond_its_scratch():
    B, cap = 4, 1 << 16
    shape = api.make_shape(B, 16, 1, 512, cap, api.LINEAR, cap)
    need = api.workspace_bytes(shape, 0, split_keys=64, impl=api.IMPL_MFMA)
    assert need > api.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 16, 512), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 1, 256, 512), dtype=torch.bfloat16, device="cuda")
    ctx = torch.ones((B,), dtype=torch.int32, device="cuda")
    out = torch.full((B, 16, 512), 7.0, device="cuda")
    with pytest.raises(api.GemmaAttnError) as e:
        # a shape whose plan needs more than the scratch (the cache tensor here is smaller
        # than the shape it is described with: nothing is launched, nothing is read)
        from decode_attention_split_amd import _lib
        import ctypes
        opts = api.make_opts(64, api.IMPL_MFMA)
        rc = _lib.load().gemma_attn_decode_noalloc(
            ctypes.byref(shape), q.data_ptr(), k.data_ptr(), None, ctx.data_ptr(),
            ctx.data_ptr(), 0, 0.0, 1.0, out.data_ptr(), ctypes.byref(opts), None)
        api._check(rc, "gemma_attn_decode_noalloc")
    assert e.value.code == -15
    torch.cuda.synchronize()
    assert (out == 7.0).all()
