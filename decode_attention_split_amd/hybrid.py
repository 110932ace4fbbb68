"""Per-layer-type KV caches for a hybrid sliding/global stack, and one decode step.

Sliding layers get a bf16 ring of W = window slots for K and for V; global (K = V)
layers get one linear bf16 tensor of C positions that serves as keys and values.  An
engine that sized every layer for the full context would silently overpay for the
sliding layers ("Gemma 4 12B (unified multimodal)" record, per-cell consequence of
missing local-attention support); here each layer's storage follows its own geometry,
the analogue of a per-layer (kv heads, head dim) table.

Every layer call goes through the C ABI (api.kv_append, api.decode); this module only
owns the tensors and the per-layer parameters.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import api
from .workloads import LINEAR, RING, LayerGeom


class HybridKVCache:
    def __init__(self, layers: List[LayerGeom], batch: int, max_ctx: int, device="cuda",
                 fill=None):
        """fill: None (torch.empty) or a callable(layer_index, name, shape) -> bf16 tensor."""
        self.layers = list(layers)
        self.batch = int(batch)
        self.max_ctx = int(max_ctx)
        self.device = torch.device(device)
        self.k: List[torch.Tensor] = []
        self.v: List[Optional[torch.Tensor]] = []
        for li, g in enumerate(self.layers):
            if g.kind == LINEAR and max_ctx > g.capacity:
                raise ValueError(f"layer {li}: max_ctx {max_ctx} exceeds linear capacity "
                                 f"{g.capacity}")
            if g.kind == RING and g.window <= 0 and max_ctx > g.capacity:
                raise ValueError(f"layer {li}: full attention on a ring needs ctx <= W")
            shape = (self.batch, g.num_kv_heads, g.capacity, g.head_dim)
            mk = (lambda name: torch.empty(shape, dtype=torch.bfloat16, device=self.device)) \
                if fill is None else (lambda name: fill(li, name, shape))
            self.k.append(mk("k"))
            self.v.append(None if g.k_eq_v else mk("v"))
        ws = 0
        for g in self.layers:
            ws = max(ws, api.workspace_bytes(self.shape(g), g.window))
        self.workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=self.device)

    def shape(self, g: LayerGeom):
        # a linear cache (or a ring without a window) never holds more than its capacity
        bounded = g.kind == LINEAR or g.window <= 0
        max_ctx = min(self.max_ctx, g.capacity) if bounded else self.max_ctx
        return api.make_shape(self.batch, g.num_q_heads, g.num_kv_heads, g.head_dim, g.capacity,
                              g.kind, max_ctx)

    def bytes(self) -> int:
        return sum(t.numel() * 2 for t in self.k) + sum(t.numel() * 2 for t in self.v
                                                           if t is not None)

    def append(self, layer: int, k_new, v_new, pos, stream=None):
        g = self.layers[layer]
        api.kv_append(self.k[layer], self.v[layer], k_new, None if g.k_eq_v else v_new, pos,
                      g.kind, stream=stream)

    def decode(self, layer: int, q, ctx_lens, q_pos, out=None, split_keys=0, impl=api.IMPL_AUTO,
               stream=None):
        g = self.layers[layer]
        return api.decode(q, self.k[layer], self.v[layer], ctx_lens, q_pos, g.window, g.softcap,
                          g.q_scale, g.kind, out=out, workspace=self.workspace,
                          max_ctx=self.shape(g).max_ctx, split_keys=split_keys, impl=impl,
                          stream=stream)

    def decode_append(self, layer: int, q, k_new, v_new, pos, ctx_lens, q_pos, out=None,
                      split_keys=0, impl=api.IMPL_AUTO, stream=None):
        """Append the new token to this layer's cache and attend, in one launch."""
        g = self.layers[layer]
        return api.decode_append(q, self.k[layer], self.v[layer], k_new,
                                 None if g.k_eq_v else v_new, pos, ctx_lens, q_pos, g.window,
                                 g.softcap, g.q_scale, g.kind, out=out, workspace=self.workspace,
                                 max_ctx=self.shape(g).max_ctx, split_keys=split_keys, impl=impl,
                                 stream=stream)

    def step(self, q_list, k_new_list, v_new_list, pos, ctx_lens, q_pos, outs, stream=None,
             fused=True):
        """One decode step through every layer: append the new token, then attend."""
        for li in range(len(self.layers)):
            if fused:
                self.decode_append(li, q_list[li], k_new_list[li], v_new_list[li], pos, ctx_lens,
                                   q_pos, out=outs[li], stream=stream)
            else:
                self.append(li, k_new_list[li], v_new_list[li], pos, stream=stream)
                self.decode(li, q_list[li], ctx_lens, q_pos, out=outs[li], stream=stream)
        return outs
