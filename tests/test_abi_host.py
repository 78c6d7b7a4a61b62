"""Host-only tests of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching a device.  Nothing
here launches a kernel or needs a GPU."""

import ctypes
import os

import pytest

from expert_ffn_layer_router_amd import _lib


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from expert_ffn_layer_router_amd import build
        build.build()
    return _lib.load()


def _cfg(**kw):
    base = dict(d_model=128, d_ff=256, num_experts=8, top_k=2, num_slots=8, max_tokens=64, flags=0)
    base.update(kw)
    return _lib.MoeConfig(**base)


def _create(lib, **kw):
    h = ctypes.c_void_p()
    st = lib.moe_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h))
    return st, h


def test_exports_every_header_function(lib):
    names = _lib.header_functions()
    assert {"moe_create", "moe_forward", "moe_graph_capture", "moe_routing_view"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_UNSUPPORTED_SHAPE"),
                       (3, "MOE_ERR_WORKSPACE_TOO_SMALL"), (4, "MOE_ERR_HIP"), (5, "MOE_ERR_BAD_STATE")]:
        assert lib.moe_status_string(code).decode() == name


@pytest.mark.parametrize("kw", [dict(d_model=100), dict(d_model=0), dict(d_ff=200), dict(num_experts=0),
                                dict(num_experts=257), dict(top_k=0), dict(top_k=9, num_experts=16),
                                dict(top_k=9, num_experts=9), dict(top_k=3, num_experts=2),
                                dict(num_slots=0), dict(max_tokens=0), dict(max_tokens=65537), dict(flags=1),
                                dict(num_shared=-1), dict(top_k=2, num_shared=7),
                                dict(num_experts=256, top_k=1, num_shared=1), dict(weight_bits=2),
                                dict(weight_bits=16), dict(group_size=64), dict(group_size=-1)])
def test_create_rejects_unsupported_shapes(lib, kw):
    st, h = _create(lib, **kw)
    assert st == _lib.MOE_ERR_UNSUPPORTED_SHAPE, _lib.last_error()
    assert not h.value
    assert _lib.last_error()


@pytest.mark.parametrize("kw", [dict(top_k=2, num_shared=6), dict(num_experts=255, top_k=1, num_shared=1),
                                dict(num_experts=1, top_k=1, num_shared=7), dict(weight_bits=8),
                                dict(weight_bits=4, group_size=128), dict(weight_bits=8, group_size=128)])
def test_create_accepts_shared_expert_limits(lib, kw):
    st, h = _create(lib, **kw)
    assert st == 0, _lib.last_error()
    lib.moe_destroy(h)


def test_shared_experts_add_rows_to_the_workspace(lib):
    """With S shared experts every token has k + S rows: the workspace grows like
    a layer with top_k + S, beyond the routed-only one.  (Token counts past 16:
    at most 16 tokens can run dense tiles, whose rows follow the experts.)"""
    sizes = {}
    for k, S in ((2, 0), (2, 2), (4, 0)):
        st, h = _create(lib, top_k=k, num_shared=S, num_experts=8, max_tokens=4096)
        assert st == 0
        n = ctypes.c_size_t()
        for T in (40, 4096):
            assert lib.moe_workspace_size(h, T, ctypes.byref(n)) == 0
            sizes[(k, S, T)] = n.value
        lib.moe_destroy(h)
    for T in (40, 4096):
        assert sizes[(2, 0, T)] < sizes[(2, 2, T)]
        # same rows as top-4, at most the few bytes of two more groups' counters apart
        assert abs(sizes[(2, 2, T)] - sizes[(4, 0, T)]) <= 2048


def test_create_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.moe_create(None, ctypes.byref(h)) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_create(ctypes.byref(_cfg()), None) == _lib.MOE_ERR_INVALID_ARG


def test_workspace_size(lib):
    st, h = _create(lib)
    assert st == 0
    sizes = []
    for T in (0, 1, 16, 64):
        n = ctypes.c_size_t()
        assert lib.moe_workspace_size(h, T, ctypes.byref(n)) == 0
        sizes.append(n.value)
    assert sizes == sorted(sizes) and sizes[-1] > sizes[0]
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(h, 65, ctypes.byref(n)) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.moe_workspace_size(h, -1, ctypes.byref(n)) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.moe_workspace_size(None, 1, ctypes.byref(n)) == _lib.MOE_ERR_INVALID_ARG
    lib.moe_destroy(h)


def test_control_bytes(lib):
    st, h = _create(lib, max_tokens=4096)
    assert st == 0
    n = ctypes.c_size_t()
    assert lib.moe_control_bytes(h, ctypes.byref(n)) == 0
    assert n.value > 0 and n.value % 256 == 0
    for T in (1, 64, 4096):  # the control words lead every workspace
        w = ctypes.c_size_t()
        assert lib.moe_workspace_size(h, T, ctypes.byref(w)) == 0
        assert n.value < w.value
    assert lib.moe_control_bytes(None, ctypes.byref(n)) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_control_bytes(h, None) == _lib.MOE_ERR_INVALID_ARG
    lib.moe_destroy(h)


FAKE = 0x10000  # an aligned address that validation never dereferences


def _forward(lib, h, T, ws_bytes=1 << 40, **over):
    w = _lib.MoeWeights(**{f: FAKE for f in ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up", "z_up",
                                            "s_down", "z_down")})
    for key in list(over):
        if hasattr(w, key):
            setattr(w, key, over.pop(key))
    args = dict(hidden=FAKE, router_w=FAKE, router_b=None, slot_table=FAKE, w=ctypes.byref(w), out=FAKE,
                ws=FAKE)
    args.update(over)
    return lib.moe_forward(h, T, args["hidden"], args["router_w"], args["router_b"], args["slot_table"],
                           args["w"], args["out"], args["ws"], ws_bytes, None)


def test_forward_validation_fails_before_enqueue(lib):
    st, h = _create(lib)
    assert st == 0
    assert _forward(lib, h, 0, hidden=None, out=None, ws=None) == _lib.MOE_OK      # T = 0: no-op
    assert _forward(lib, h, 65) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert _forward(lib, h, -1) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert _forward(lib, h, 4, hidden=None) == _lib.MOE_ERR_INVALID_ARG
    assert _forward(lib, h, 4, w=None) == _lib.MOE_ERR_INVALID_ARG
    assert _forward(lib, h, 4, s_down=None) == _lib.MOE_ERR_INVALID_ARG
    assert _forward(lib, h, 4, hidden=FAKE + 2) == _lib.MOE_ERR_INVALID_ARG        # misaligned
    assert _forward(lib, h, 4, w_up=FAKE + 8) == _lib.MOE_ERR_INVALID_ARG
    assert _forward(lib, h, 4, slot_table=FAKE + 1) == _lib.MOE_ERR_INVALID_ARG
    assert _forward(lib, h, 4, ws_bytes=1) == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    assert "needs" in _lib.last_error()
    assert lib.moe_forward(None, 4, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 1 << 40, None) \
        == _lib.MOE_ERR_INVALID_ARG
    lib.moe_destroy(h)


def test_graph_launch_without_capture_is_bad_state(lib):
    st, h = _create(lib)
    assert lib.moe_graph_launch(h, None) == _lib.MOE_ERR_BAD_STATE
    lib.moe_destroy(h)


def test_routing_view_is_pointer_arithmetic(lib):
    st, h = _create(lib, max_tokens=32)
    v = _lib.MoeRouting()
    base = 1 << 32
    assert lib.moe_routing_view(h, base, 16, ctypes.byref(v)) == 0
    ptrs = [v.topk_idx, v.topk_w, v.counts, v.offsets, v.perm, v.inv_perm]
    assert all(p >= base for p in ptrs) and len(set(ptrs)) == 6
    assert all((p - base) % 256 == 0 for p in ptrs)
    n = ctypes.c_size_t()
    lib.moe_workspace_size(h, 16, ctypes.byref(n))
    assert all(p - base < n.value for p in ptrs)
    assert lib.moe_routing_view(h, base, 33, ctypes.byref(v)) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    lib.moe_destroy(h)


def test_destroy_tolerates_null(lib):
    lib.moe_destroy(None)
