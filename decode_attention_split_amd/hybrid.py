"""Per-layer-type KV caches for a hybrid sliding/global stack, and one decode step.

Sliding layers get a bf16 ring of W = window slots for K and for V; global (K = V)
layers get one linear bf16 tensor of C positions that serves as keys and values.  An
engine that sized every layer for the full context would silently overpay for the
sliding layers ("Gemma 4 12B (unified multimodal)" record, per-cell consequence of
missing local-attention support); here each layer's storage follows its own geometry,
the analogue of a per-layer (kv heads, head dim) table.

Layers may share a cache (num_kv_shared_layers, "Gemma 4 12B (unified multimodal)"
record, "KV geometry, now derived"): a sharing layer holds no tensors of its own, never
appends, and attends over its owner's cache, which the owner has already extended with
the step's token.

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
                 fill=None, kv_source: Optional[List[int]] = None):
        """fill: None (torch.empty) or a callable(layer_index, name, shape) -> bf16 tensor.
        kv_source: per layer, the index of the layer whose cache it reads (default: its
        own); see workloads.kv_share_sources."""
        self.layers = list(layers)
        self.batch = int(batch)
        self.max_ctx = int(max_ctx)
        self.device = torch.device(device)
        n = len(self.layers)
        self.kv_source = list(range(n)) if kv_source is None else [int(s) for s in kv_source]
        if len(self.kv_source) != n:
            raise ValueError("kv_source needs one entry per layer")
        for li, src in enumerate(self.kv_source):
            if src != li and (not 0 <= src < li or self.kv_source[src] != src
                              or self.layers[src] != self.layers[li]):
                raise ValueError(f"layer {li}: must share the cache of an earlier owner layer "
                                 f"of the same geometry (got {src})")
        self.k: List[torch.Tensor] = []
        self.v: List[Optional[torch.Tensor]] = []
        for li, g in enumerate(self.layers):
            if g.kind == LINEAR and max_ctx > g.capacity:
                raise ValueError(f"layer {li}: max_ctx {max_ctx} exceeds linear capacity "
                                 f"{g.capacity}")
            if g.kind == RING and g.window <= 0 and max_ctx > g.capacity:
                raise ValueError(f"layer {li}: full attention on a ring needs ctx <= W")
            src = self.kv_source[li]
            if src != li:  # shares the owner's tensors
                self.k.append(self.k[src])
                self.v.append(self.v[src])
                continue
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

    def owns_cache(self, layer: int) -> bool:
        return self.kv_source[layer] == layer

    def bytes(self) -> int:
        """Bytes of cache storage (shared caches counted once)."""
        owners = [i for i in range(len(self.layers)) if self.owns_cache(i)]
        return sum(self.k[i].numel() * 2 for i in owners) + \
            sum(self.v[i].numel() * 2 for i in owners if self.v[i] is not None)

    def append(self, layer: int, k_new, v_new, pos, stream=None):
        if not self.owns_cache(layer):
            raise ValueError(f"layer {layer} shares layer {self.kv_source[layer]}'s cache and "
                             "does not append")
        g = self.layers[layer]
        api.kv_append(self.k[layer], self.v[layer], k_new, None if g.k_eq_v else v_new, pos,
                      g.kind, stream=stream)

    def decode(self, layer: int, q, ctx_lens, q_pos, out=None, split_keys=0, impl=api.IMPL_AUTO,
               deterministic=False, stream=None):
        g = self.layers[layer]
        return api.decode(q, self.k[layer], self.v[layer], ctx_lens, q_pos, g.window, g.softcap,
                          g.q_scale, g.kind, out=out, workspace=self.workspace,
                          max_ctx=self.shape(g).max_ctx, split_keys=split_keys, impl=impl,
                          deterministic=deterministic, stream=stream)

    def decode_append(self, layer: int, q, k_new, v_new, pos, ctx_lens, q_pos, out=None,
                      split_keys=0, impl=api.IMPL_AUTO, deterministic=False, stream=None):
        """Append the new token to this layer's cache and attend, in one launch.  A layer
        that shares another's cache only attends (its owner appended the token)."""
        g = self.layers[layer]
        if not self.owns_cache(layer):
            return self.decode(layer, q, ctx_lens, q_pos, out=out, split_keys=split_keys,
                               impl=impl, deterministic=deterministic, stream=stream)
        return api.decode_append(q, self.k[layer], self.v[layer], k_new,
                                 None if g.k_eq_v else v_new, pos, ctx_lens, q_pos, g.window,
                                 g.softcap, g.q_scale, g.kind, out=out, workspace=self.workspace,
                                 max_ctx=self.shape(g).max_ctx, split_keys=split_keys, impl=impl,
                                 deterministic=deterministic, stream=stream)

    def rope_append(self, layer: int, q, q_out, k_new, v_new, pos, stream=None):
        """Rotary embedding of q (-> q_out) and of the new K row, fused with the append (a
        layer that shares another's cache only rotates q)."""
        g = self.layers[layer]
        if not self.owns_cache(layer):
            return api.rope_append(q, q_out, None, None, None, None, pos, g.kind, g.rope_base,
                                   g.rotary_dim, stream=stream)
        return api.rope_append(q, q_out, self.k[layer], self.v[layer], k_new,
                               None if g.k_eq_v else v_new, pos, g.kind, g.rope_base,
                               g.rotary_dim, stream=stream)

    def rope_tables(self, pos, stream=None):
        """cos / sin tables at pos, one per (base, rotary_dim, head_dim) among the rotary
        layers, keyed by that triple; every layer of a type reads its type's table."""
        tables = {}
        for g in self.layers:
            key = (g.rope_base, g.rotary_dim, g.head_dim)
            if g.rope_base > 0 and key not in tables:
                tables[key] = api.rope_table(pos, g.rope_base, g.rotary_dim, g.head_dim,
                                             stream=stream)
        return tables

    def decode_rope_append(self, layer: int, q, q_out, k_new, v_new, pos, ctx_lens, q_pos,
                           table, out=None, deterministic=False, stream=None):
        """Rotary embedding, append and decode of a cache-owning layer in one call (one
        launch on the vector kernel, and on the global matrix-core kernel when q_out is a
        buffer of its own); table from rope_tables(pos)."""
        g = self.layers[layer]
        if not self.owns_cache(layer):
            raise ValueError(f"layer {layer} shares layer {self.kv_source[layer]}'s cache and "
                             "does not append")
        return api.decode_rope_append(q, q_out, self.k[layer], self.v[layer], k_new,
                                      None if g.k_eq_v else v_new, pos, ctx_lens, q_pos,
                                      g.window, g.softcap, g.q_scale, g.kind, table,
                                      g.rotary_dim, out=out, workspace=self.workspace,
                                      max_ctx=self.shape(g).max_ctx, deterministic=deterministic,
                                      stream=stream)

    def step(self, q_list, k_new_list, v_new_list, pos, ctx_lens, q_pos, outs, stream=None,
             fused=True, deterministic=False, q_rot=None):
        """One decode step through every layer: append the new token, then attend.  Layers
        with a rotary embedding (rope_base > 0) rotate q (into q_rot[layer], or in place when
        q_rot is None) and the new K row before the append; with fused, a cache-owning layer
        does all of it in one call, on the step's cos / sin table of its layer type."""
        tables = self.rope_tables(pos, stream=stream) if fused else {}
        for li in range(len(self.layers)):
            g = self.layers[li]
            if g.rope_base > 0:
                qo = q_list[li] if q_rot is None else q_rot[li]
                if fused and self.owns_cache(li):
                    self.decode_rope_append(li, q_list[li], qo, k_new_list[li], v_new_list[li],
                                            pos, ctx_lens, q_pos,
                                            tables[(g.rope_base, g.rotary_dim, g.head_dim)],
                                            out=outs[li],
                                            deterministic=deterministic, stream=stream)
                    continue
                self.rope_append(li, q_list[li], qo, k_new_list[li], v_new_list[li], pos,
                                 stream=stream)
                self.decode(li, qo, ctx_lens, q_pos, out=outs[li], deterministic=deterministic,
                            stream=stream)
                continue
            if fused:
                self.decode_append(li, q_list[li], k_new_list[li], v_new_list[li], pos, ctx_lens,
                                   q_pos, out=outs[li], deterministic=deterministic,
                                   stream=stream)
            else:
                if self.owns_cache(li):
                    self.append(li, k_new_list[li], v_new_list[li], pos, stream=stream)
                self.decode(li, q_list[li], ctx_lens, q_pos, out=outs[li],
                            deterministic=deterministic, stream=stream)
        return outs
