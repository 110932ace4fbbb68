"""Decode-attention workloads: the per-layer geometries of Gemma-3/4-style hybrid stacks.

Geometry sources (page titles and sections):
  * "Gemma 4 12B (unified multimodal)" record, "KV geometry, now derived" and the
    layer_types passage: 40 sliding layers with 8 KV heads of head_dim 256, 8 full
    layers with 1 KV head of global_head_dim 512, full layers at 0-based indices
    5, 11, ..., 47, attention_k_eq_v true, bounded sliding window.
  * "Gemma4-26B-A4B on Apple Silicon", Results (Break 4): per-layer-type head dims and
    KV-head counts; K/V sharing on full layers.  Threats to validity: the query scale
    defaults to 1/sqrt(head_dim) per geometry.
  * "Gemma support" pull request, Summary: soft-capping, sliding-window layers, mixed
    256/512 head sizes, K = V global attention; Test plan: kernel tests over head sizes
    128 to 512.
  * "Gemma 4 12B (unified multimodal)" record, "KV geometry, now derived":
    num_kv_shared_layers (0 for that model) counts layers that take a neighbour's cache
    instead of keeping their own.

Nothing here computes attention; these are shapes, seeds and counts.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

LINEAR = 0
RING = 1


def default_scale(head_dim: int) -> float:
    """float32(1/sqrt(head_dim)): the default query pre-attention scale."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


@dataclass(frozen=True)
class LayerGeom:
    """One attention layer's decode geometry."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kind: int            # LINEAR or RING
    capacity: int        # ring: W slots; linear: C positions
    window: int          # <= 0: full causal
    k_eq_v: bool         # one cached tensor serves as keys and values
    softcap: float = 0.0  # <= 0: off
    scale: Optional[float] = None  # None: 1/sqrt(head_dim)
    rope_base: float = 0.0  # > 0: rotary embedding applied by the step (base)
    rotary_dim: int = 0     # rotated width R (even): pairs (i, i + D/2), i < R/2, turn

    @property
    def q_scale(self) -> float:
        return default_scale(self.head_dim) if self.scale is None else float(np.float32(self.scale))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_token(self, count_v_for_k_eq_v: bool = False) -> int:
        """bf16 bytes one token adds to this layer's cache (K, plus V unless K = V)."""
        tensors = 1 if (self.k_eq_v and not count_v_for_k_eq_v) else 2
        return self.num_kv_heads * self.head_dim * tensors * 2


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    ctx_lo: int
    ctx_hi: int
    layers: List[LayerGeom] = field(default_factory=list)
    tokens: int = 1  # query tokens per row (T > 1: multi-token decode)
    kv_dtype: str = "bf16"  # "bf16" or "fp8" (e4m3 codes + float32 row scales)

    @property
    def num_layers(self) -> int:
        return len(self.layers)


def sliding_geom(num_q, num_kv, window, softcap=0.0, scale=None, head_dim=256):
    return LayerGeom(num_q, num_kv, head_dim, RING, window, window, False, softcap, scale)


def global_geom(num_q, capacity, head_dim=512, num_kv=1, softcap=0.0, scale=None):
    return LayerGeom(num_q, num_kv, head_dim, LINEAR, capacity, 0, True, softcap, scale)


def with_rope(g: LayerGeom, base: float, rotary_dim: int) -> LayerGeom:
    return replace(g, rope_base=float(base), rotary_dim=int(rotary_dim))


# Rotary embedding per layer type: sliding layers base 10,000 over the whole head, full
# layers base 1,000,000 on the low part of the head ("Gemma support" pull request, Summary;
# "Gemma4-26B-A4B on Apple Silicon", Results (Break 4) and Ablations / negative controls;
# the model-loader page's header).  The pages do not give the rotated fraction of a full
# layer's head; a quarter (128 of 512) is this reading.
SLIDING_ROPE_BASE, GLOBAL_ROPE_BASE = 1e4, 1e6
GLOBAL_ROTARY_FRACTION = 4


def gemma4_12b_layer_types(num_layers: int = 48, period: int = 6) -> List[str]:
    """Layer schedule: full attention at 0-based index l when l % period == period - 1."""
    return ["full_attention" if (l % period) == period - 1 else "sliding_attention"
            for l in range(num_layers)]


def hybrid_layers(num_layers=48, sliding=None, full=None) -> List[LayerGeom]:
    sliding = sliding or sliding_geom(16, 8, 1024)
    full = full or global_geom(16, 16384)
    return [full if t == "full_attention" else sliding for t in gemma4_12b_layer_types(num_layers)]


def kv_share_sources(layers: List[LayerGeom], num_kv_shared_layers: int = 0) -> List[int]:
    """Index of the layer whose cache each layer reads (itself when it owns one).

    Reading of num_kv_shared_layers (the pages name the field, and say that a layer
    sharing cache takes it from a neighbour): the last N layers of the stack keep no
    cache; each reads the cache of the nearest earlier non-shared layer with the same
    geometry.  Those owners come first in the stack, so within one step an owner has
    appended the token before any layer that shares its cache attends.
    """
    n = len(layers)
    if not 0 <= num_kv_shared_layers < n:
        raise ValueError(f"num_kv_shared_layers must be in [0, {n})")
    first_shared = n - num_kv_shared_layers
    src = list(range(n))
    for l in range(first_shared, n):
        owners = [o for o in range(first_shared) if layers[o] == layers[l]]
        if not owners:
            raise ValueError(f"layer {l}: no earlier layer with the same geometry to share")
        src[l] = owners[-1]
    return src


def kv_bytes_per_token(layers: List[LayerGeom], count_v_for_k_eq_v: bool = False,
                       sources: Optional[List[int]] = None) -> int:
    """Cache bytes one token adds across the stack; layers that share a cache add none."""
    owners = range(len(layers)) if sources is None else sorted(set(sources))
    return sum(layers[i].kv_bytes_per_token(count_v_for_k_eq_v) for i in owners)


# The five synthetic workloads (seed = index).
TINY = Workload("tiny sliding decode, B1 4q/1kv hd256 ctx64 ring w32 softcap50", 1, 1, 64, 64,
                [sliding_geom(4, 1, 32, softcap=50.0, scale=1.0 / 16)])
G3_1B_SLIDING = Workload("gemma3-1b sliding layer, B32 4q/1kv hd256 ring w512 ctx U[1,1024]", 2, 32,
                         1, 1024, [sliding_geom(4, 1, 512, scale=1.0 / 16)])
G4_12B_SLIDING = Workload("gemma4-12b sliding layer, B64 16q/8kv hd256 ring w1024 ctx U[512,8192]"
                          " softcap50", 3, 64, 512, 8192,
                          [sliding_geom(16, 8, 1024, softcap=50.0, scale=1.0 / 16)])
G4_12B_GLOBAL = Workload("gemma4-12b global layer, B16 16q/1kv K=V hd512 linear C32768"
                         " ctx U[4096,32768]", 4, 16, 4096, 32768, [global_geom(16, 32768)])
HYBRID_48 = Workload("48-layer hybrid decode step, B32 ctx U[1,16384]: 40 sliding (16q/8kv hd256"
                     " ring w1024) + 8 global (16q/1kv K=V hd512 linear C16384)", 5, 32, 1, 16384,
                     hybrid_layers(48, sliding_geom(16, 8, 1024), global_geom(16, 16384)))

ALL = [TINY, G3_1B_SLIDING, G4_12B_SLIDING, G4_12B_GLOBAL, HYBRID_48]

# The 48-layer step with the rotary embedding fused into each layer's append.
HYBRID_48_ROPE = replace(
    HYBRID_48, name=HYBRID_48.name + "; rotary embedding fused with the append (sliding base "
    "1e4 over 256, global base 1e6 over 128)",
    layers=hybrid_layers(48, with_rope(sliding_geom(16, 8, 1024), SLIDING_ROPE_BASE, 256),
                         with_rope(global_geom(16, 16384), GLOBAL_ROPE_BASE,
                                   512 // GLOBAL_ROTARY_FRACTION)))

# Extra single-layer workloads for the head sizes the kernel tests span (128 to 512):
# the long-context sliding layer of the 12B geometry at head_dim 128.
HD128_SLIDING = Workload("hd128 sliding layer, B64 16q/8kv hd128 ring w1024 ctx U[512,8192]"
                         " softcap50", 6, 64, 512, 8192,
                         [sliding_geom(16, 8, 1024, softcap=50.0, head_dim=128)])

# The 12B sliding layer over an fp8 cache (e4m3 codes, one float32 scale per row): half
# the bytes per key (the fp8_e4m3 KV cache of the "Gemma 4 12B (unified multimodal)"
# record, item "(2)").
FP8_SLIDING = replace(G4_12B_SLIDING, name="gemma4-12b sliding layer, fp8 e4m3 cache with "
                      "per-row scales, B64 16q/8kv hd256 ring w1024 ctx U[512,8192] softcap50",
                      seed=8, kv_dtype="fp8")

# The 12B global layer (K = V, hd512, 16 query heads on one KV head) over an fp8 cache:
# the matrix-core kernel widens the codes to bf16 in registers.
FP8_GLOBAL = replace(G4_12B_GLOBAL, name="gemma4-12b global layer, fp8 e4m3 cache with per-row "
                     "scales, B16 16q/1kv K=V hd512 linear C32768 ctx U[4096,32768]", seed=10,
                     kv_dtype="fp8")

# Speculative verification on the 12B sliding layer: 7 draft tokens plus the current one
# (T = 8, the k = 7 spec decode of the "Gemma 4 12B (unified multimodal)" record, item
# "(2)"), each masked at its own position.  The ring keeps w + T - 1 = 1031 slots so the
# first token's window is still present.
SPEC_DECODE_SLIDING = Workload("gemma4-12b sliding layer verifying 7 draft tokens (T=8), B64 "
                               "16q/8kv hd256 ring W=1031 w1024 ctx U[512,8192] softcap50", 7,
                               64, 512, 8192,
                               [LayerGeom(16, 8, 256, RING, 1031, 1024, False, 50.0, 1.0 / 16)],
                               tokens=8)


# The same verification over an fp8 cache: BF16 queries with FP8 KV and spec decode on a
# sliding window, the combination item "(2)" of the "Gemma 4 12B (unified multimodal)"
# record reports as corrupting in another engine.
FP8_SPEC_DECODE_SLIDING = replace(SPEC_DECODE_SLIDING, name="gemma4-12b sliding layer verifying "
                                  "7 draft tokens (T=8) over an fp8 e4m3 cache, B64 16q/8kv "
                                  "hd256 ring W=1031 w1024 ctx U[512,8192] softcap50", seed=11,
                                  kv_dtype="fp8")

def layer_seed(workload: Workload, layer: int) -> int:
    """Per-layer seed of a multi-layer workload (single-layer workloads use the seed)."""
    return workload.seed if workload.num_layers == 1 else workload.seed * 1000 + layer


def with_batch(w: Workload, batch: int) -> Workload:
    return replace(w, batch=batch)
