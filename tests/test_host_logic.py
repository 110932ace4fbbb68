"""CPU: host-side logic around the kernels (layer schedule, cache sharing, cache objects).

No compute call is made here; HybridKVCache is built on the CPU, which only allocates
tensors and asks the library (host code) for workspace sizes.
"""
import pytest
import torch

from decode_attention_split_amd import workloads as wl
from decode_attention_split_amd.hybrid import HybridKVCache


def test_share_sources_default_is_own_cache():
    layers = wl.hybrid_layers(48)
    assert wl.kv_share_sources(layers, 0) == list(range(48))


def test_share_sources_take_nearest_earlier_owner_of_same_type():
    # 12 layers, global at 5 and 11; the last 4 (8..11) share: sliding 8, 9, 10 take
    # sliding 7, global 11 takes global 5
    layers = wl.hybrid_layers(12)
    src = wl.kv_share_sources(layers, 4)
    assert src == [0, 1, 2, 3, 4, 5, 6, 7, 7, 7, 7, 5]
    for l, s in enumerate(src):
        assert layers[l] == layers[s] and s <= l and src[s] == s


def test_share_sources_rejects_a_layer_without_an_owner():
    layers = [wl.sliding_geom(16, 8, 1024), wl.global_geom(16, 4096)]
    with pytest.raises(ValueError):
        wl.kv_share_sources(layers, 1)  # the global layer has no earlier global owner
    with pytest.raises(ValueError):
        wl.kv_share_sources(layers, 2)


def test_bytes_per_token_counts_shared_caches_once():
    layers = wl.hybrid_layers(12)
    sliding, full = layers[0], layers[5]
    src = wl.kv_share_sources(layers, 4)
    # owners: sliding 0-4, 6, 7 (7 layers) and global 5: 7 * 8*256*2*2 + 1 * 1*512*2
    assert wl.kv_bytes_per_token(layers, sources=src) == 7 * 8192 + 1024
    assert wl.kv_bytes_per_token(layers) == 10 * 8192 + 2 * 1024
    assert sliding.kv_bytes_per_token() == 8192 and full.kv_bytes_per_token() == 1024


def test_hybrid_cache_aliases_shared_layers():
    layers = wl.hybrid_layers(12, wl.sliding_geom(4, 2, 64), wl.global_geom(4, 256, num_kv=1))
    src = wl.kv_share_sources(layers, 4)
    cache = HybridKVCache(layers, 2, 256, device="cpu", kv_source=src)
    for l, s in enumerate(src):
        assert cache.k[l].data_ptr() == cache.k[s].data_ptr()
        assert cache.owns_cache(l) == (l == s)
    own = HybridKVCache(layers, 2, 256, device="cpu")
    per_sliding = 2 * 2 * 64 * 256 * 2 * 2
    per_global = 2 * 1 * 256 * 512 * 2
    assert own.bytes() == 10 * per_sliding + 2 * per_global
    assert cache.bytes() == 7 * per_sliding + 1 * per_global
    with pytest.raises(ValueError):
        cache.append(9, None, None, None)  # a sharing layer never appends


def test_hybrid_cache_rejects_bad_sharing():
    layers = wl.hybrid_layers(12, wl.sliding_geom(4, 2, 64), wl.global_geom(4, 256, num_kv=1))
    bad = list(range(12))
    bad[3] = 5  # sliding layer pointing at a global one
    with pytest.raises(ValueError):
        HybridKVCache(layers, 1, 256, device="cpu", kv_source=bad)
    bad = list(range(12))
    bad[2] = 4  # a later layer
    with pytest.raises(ValueError):
        HybridKVCache(layers, 1, 256, device="cpu", kv_source=bad)


def test_hd128_workload_geometry():
    w = wl.HD128_SLIDING
    g = w.layers[0]
    assert (g.head_dim, g.num_q_heads, g.num_kv_heads, g.capacity, g.window) == (128, 16, 8, 1024,
                                                                                1024)
    assert g.q_scale == pytest.approx(1 / 128 ** 0.5, rel=1e-7)
