"""The library's expert cache (host code, no device call) against the plain
model in oracle/expert_cache.py: the same slots, loads, slot tables and hit
counts on random request streams, and the same errors."""

import random

import pytest

from oracle.expert_cache import ExpertCacheModel
from expert_ffn_layer_router_amd import _lib
from expert_ffn_layer_router_amd.layer import ExpertCache


@pytest.fixture(scope="module", autouse=True)
def _built():
    import os
    if not os.path.exists(_lib.LIB_PATH):
        from expert_ffn_layer_router_amd import build
        build.build()


@pytest.mark.parametrize("seed", range(8))
def test_library_cache_matches_the_model(seed):
    rng = random.Random(100 + seed)
    num_sets, ways, E, L = rng.choice([1, 2, 5]), rng.choice([1, 2, 4, 8]), rng.choice([8, 16, 64]), 7
    lib_cache, model = ExpertCache(num_sets, ways, E), ExpertCacheModel(num_sets, ways, E)
    for _ in range(400):
        layer = rng.randrange(L)
        experts = [rng.randrange(E) for _ in range(rng.randint(1, ways))]
        slots, loads, table = lib_cache.request(layer, experts)
        mslots, mloads = model.request(layer, experts)
        assert (slots, loads) == (mslots, mloads)
        assert table == model.slot_table(layer)
    assert lib_cache.stats() == (model.hits, model.misses)


def test_rejected_requests_leave_the_cache_unchanged():
    c = ExpertCache(1, 2, 8)
    c.request(0, [1, 2])
    with pytest.raises(_lib.MoeError):
        c.request(0, [3, 4, 5])          # three distinct experts, two ways
    with pytest.raises(_lib.MoeError):
        c.request(0, [8])                # expert out of range
    with pytest.raises(_lib.MoeError):
        c.request(-1, [0])               # negative layer
    assert c.request(0, [1, 2]) == ([0, 1], [], [-1, 0, 1, -1, -1, -1, -1, -1])
    assert c.stats() == (2, 2)


def test_create_rejects_bad_shapes():
    lib = _lib.load()
    import ctypes
    h = ctypes.c_void_p()
    for args in ((0, 4, 8), (2, 0, 8), (2, 4, 0), (1 << 13, 1 << 12, 8)):
        assert lib.moe_cache_create(*args, ctypes.byref(h)) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_cache_create(2, 4, 8, None) == _lib.MOE_ERR_INVALID_ARG


def test_library_geometry_matches_the_model():
    from oracle.expert_cache import cache_geometry
    rng = random.Random(9)
    for _ in range(200):
        free = rng.randrange(0, 1 << 40)
        expert = rng.randrange(1 << 20, 1 << 32)
        ways = rng.randint(1, 16)
        assert ExpertCache.geometry(free, expert, ways) == cache_geometry(free, expert, ways)
    assert ExpertCache.geometry(19 << 30, 340 << 20, 4) == (57, 14)
    with pytest.raises(_lib.MoeError):
        ExpertCache.geometry(1 << 30, 0, 4)
    with pytest.raises(_lib.MoeError):
        ExpertCache.geometry(1 << 30, 1 << 20, 0)


@pytest.mark.parametrize("bits,group", [(4, 0), (4, 128), (8, 0), (8, 128)])
def test_expert_bytes_is_the_size_of_one_pool_slot(bits, group):
    """moe_expert_bytes == the bytes of one slot of the synthetic pool arrays."""
    import synth
    from expert_ffn_layer_router_amd import MoeLayer
    shape = synth.LayerShape(4, 256, 384, 4, 2, 4, "identity", 0.0, 0, bits, group)
    w = synth.make_weights(shape, seed=1)
    layer = MoeLayer(256, 384, 4, 2, 4, 4, weight_bits=bits, group_size=group)
    per_slot = sum(getattr(w, f)[0].nbytes for f in ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up",
                                                     "z_up", "s_down", "z_down"))
    assert layer.expert_bytes() == per_slot
