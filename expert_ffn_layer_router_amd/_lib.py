"""ctypes declarations of the C ABI in include/moe.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import glob
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_hip.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADERS = sorted(glob.glob(os.path.join(INCLUDE, "*.h")))

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED_SHAPE = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4
MOE_ERR_BAD_STATE = 5
MOE_FLAG_BAD_SLOT = 0x1
MOE_NUM_STAGES = 5
STAGE_NAMES = ("router", "regroup", "gate_up", "down", "combine")


class MoeConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("num_slots", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("num_shared", ctypes.c_int32), ("weight_bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up", "z_up", "s_down", "z_down")]


class MoeRouting(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm")]


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


_lib = None


def header_functions() -> list:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for path in HEADERS:
        with open(path) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def load():
    """The in-tree libmoe_hip.so.  Raises if it has not been built: there is no
    fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m expert_ffn_layer_router_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    i32 = ctypes.c_int32
    sig = {
        "moe_create": (c_int, [ctypes.POINTER(MoeConfig), ctypes.POINTER(vp)]),
        "moe_destroy": (None, [vp]),
        "moe_workspace_size": (c_int, [vp, i32, ctypes.POINTER(sz)]),
        "moe_control_bytes": (c_int, [vp, ctypes.POINTER(sz)]),
        "moe_cache_create": (c_int, [i32, i32, i32, ctypes.POINTER(vp)]),
        "moe_cache_destroy": (None, [vp]),
        "moe_cache_request": (c_int, [vp, i32, vp, i32, vp, vp, vp, ctypes.POINTER(i32), vp]),
        "moe_cache_stats": (c_int, [vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
        "moe_expert_upload": (c_int, [vp, ctypes.POINTER(MoeWeights), i32, ctypes.POINTER(MoeWeights), vp]),
        "moe_cache_geometry": (c_int, [ctypes.c_uint64, ctypes.c_uint64, i32, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_int32)]),
        "moe_expert_bytes": (c_int, [vp, ctypes.POINTER(ctypes.c_uint64)]),
        "moe_forward": (c_int, [vp, i32, vp, vp, vp, vp, ctypes.POINTER(MoeWeights), vp, vp, sz, vp]),
        "moe_forward_noalloc": (c_int, [vp, i32, vp, vp, vp, vp, ctypes.POINTER(MoeWeights), vp, vp]),
        "moe_routing_view": (c_int, [vp, vp, i32, ctypes.POINTER(MoeRouting)]),
        "moe_graph_capture": (c_int, [vp, i32, vp, vp, vp, vp, ctypes.POINTER(MoeWeights), vp, vp, sz, vp]),
        "moe_graph_launch": (c_int, [vp, vp]),
        "moe_device_flags": (c_int, [vp, vp, i32, vp, ctypes.POINTER(ctypes.c_uint32)]),
        "moe_set_stage_timing": (c_int, [vp, i32]),
        "moe_stage_times": (c_int, [vp, ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]),
        "moe_hbm_read_probe": (c_int, [vp, sz, vp, i32, vp]),
        "moe_status_string": (ctypes.c_char_p, [c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def last_error() -> str:
    return load().moe_last_error().decode()


def check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, last_error())
