"""Python face of the C ABI.  torch supplies device memory and the stream;
every step of the layer runs in the library's HIP kernels."""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np

from . import _lib

WEIGHT_FIELDS = ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up", "z_up", "s_down", "z_down")


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def to_device(arr: np.ndarray, device="cuda"):
    """numpy -> torch on `device`; uint16 arrays keep their bit patterns (int16)."""
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


@dataclasses.dataclass
class DeviceWeights:
    """The slot-indexed weight pool (codes, scales, zero-points) on the device
    (keeps the tensors alive)."""
    tensors: dict

    @classmethod
    def upload(cls, weights, device="cuda") -> "DeviceWeights":
        src = weights if isinstance(weights, dict) else {f: getattr(weights, f) for f in WEIGHT_FIELDS}
        return cls({f: to_device(src[f], device) for f in WEIGHT_FIELDS})

    def struct(self) -> _lib.MoeWeights:
        return _lib.MoeWeights(**{f: _ptr(self.tensors[f]) for f in WEIGHT_FIELDS})

    def clone(self) -> "DeviceWeights":
        """A second copy of the pool in device memory (device-to-device copies)."""
        return DeviceWeights({f: t.clone() for f, t in self.tensors.items()})


def hbm_read_probe(buf, sink, blocks: int = 2048, stream=None) -> None:
    """moe_hbm_read_probe: one read of the device tensor `buf`, XOR-folded into
    the int32 device tensor `sink` (measurement yardstick)."""
    torch = _torch()
    lib = _lib.load()
    s = torch.cuda.current_stream() if stream is None else stream
    _lib.check(lib.moe_hbm_read_probe(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(sink), int(blocks),
                                      ctypes.c_void_p(int(s.cuda_stream))))


class MoeLayer:
    """One layer shape.  Mirrors moe_create / moe_forward / moe_routing_view /
    moe_graph_capture / moe_graph_launch / moe_device_flags."""

    def __init__(self, d_model: int, d_ff: int, num_experts: int, top_k: int, num_slots: int,
                 max_tokens: int, num_shared: int = 0, weight_bits: int = 4, group_size: int = 0):
        self.lib = _lib.load()
        self.cfg = _lib.MoeConfig(d_model, d_ff, num_experts, top_k, num_slots, max_tokens, 0, num_shared,
                                  weight_bits, group_size)
        h = ctypes.c_void_p()
        _lib.check(self.lib.moe_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self.handle = h
        self._graph_keepalive = None

    def close(self):
        if getattr(self, "handle", None):
            self.lib.moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, T: int) -> int:
        n = ctypes.c_size_t()
        _lib.check(self.lib.moe_workspace_size(self.handle, int(T), ctypes.byref(n)))
        return n.value

    def control_bytes(self) -> int:
        """Bytes at the start of a workspace holding control words (kept zero)."""
        n = ctypes.c_size_t()
        _lib.check(self.lib.moe_control_bytes(self.handle, ctypes.byref(n)))
        return n.value

    def new_workspace(self, T: int, device="cuda"):
        """A zero-filled workspace (the library's control words must start at zero)."""
        torch = _torch()
        return torch.zeros(max(self.workspace_size(T), 256), dtype=torch.uint8, device=device)

    @staticmethod
    def _stream(stream):
        torch = _torch()
        s = torch.cuda.current_stream() if stream is None else stream
        return ctypes.c_void_p(int(s.cuda_stream))

    def _args(self, hidden, router_w, router_b, slot_table, weights, out, workspace):
        T = int(hidden.shape[0])
        return (self.handle, T, _ptr(hidden), _ptr(router_w), _ptr(router_b), _ptr(slot_table),
                ctypes.byref(weights.struct()), _ptr(out), _ptr(workspace),
                int(workspace.numel() * workspace.element_size()))

    def forward(self, hidden, router_w, router_b, slot_table, weights: DeviceWeights, out=None,
                workspace=None, stream=None):
        """hidden: bf16 (or int16 bit patterns) [T, d] on the device.  Returns out [T, d]."""
        torch = _torch()
        T = int(hidden.shape[0])
        if out is None:
            out = torch.empty((T, self.cfg.d_model), dtype=hidden.dtype, device=hidden.device)
        if workspace is None:
            workspace = self.new_workspace(T, hidden.device)
        _lib.check(self.lib.moe_forward(*self._args(hidden, router_w, router_b, slot_table, weights, out,
                                                    workspace), self._stream(stream)))
        return out

    def forward_noalloc(self, hidden, router_w, router_b, slot_table, weights: DeviceWeights, out, stream=None):
        """moe_forward_noalloc: the forward with the library's own device scratch
        instead of a workspace (calls on one device must not overlap).  `out`
        [T, d] is the caller's."""
        T = int(hidden.shape[0])
        _lib.check(self.lib.moe_forward_noalloc(self.handle, T, _ptr(hidden), _ptr(router_w), _ptr(router_b),
                                                _ptr(slot_table), ctypes.byref(weights.struct()), _ptr(out),
                                                self._stream(stream)))
        return out

    def capture(self, hidden, router_w, router_b, slot_table, weights: DeviceWeights, out, workspace,
                stream):
        """Captures a forward into the handle's graph (buffers must outlive the graph)."""
        _lib.check(self.lib.moe_graph_capture(*self._args(hidden, router_w, router_b, slot_table, weights,
                                                          out, workspace), self._stream(stream)))
        self._graph_keepalive = (hidden, router_w, router_b, slot_table, weights, out, workspace)

    def replay(self, stream=None):
        _lib.check(self.lib.moe_graph_launch(self.handle, self._stream(stream)))

    def routing(self, workspace, T: int) -> dict:
        """Views (into `workspace`) of the routing the last forward left there."""
        torch = _torch()
        v = _lib.MoeRouting()
        _lib.check(self.lib.moe_routing_view(self.handle, _ptr(workspace), int(T), ctypes.byref(v)))
        base = int(workspace.data_ptr())
        # shared experts are extra columns of every token and extra groups
        k = self.cfg.top_k + self.cfg.num_shared
        E = self.cfg.num_experts + self.cfg.num_shared
        R = int(T) * k

        def view(ptr, n, dtype):
            off = int(ptr) - base
            return workspace[off:off + 4 * n].view(dtype)

        return dict(topk_idx=view(v.topk_idx, R, torch.int32).view(int(T), k),
                    topk_w=view(v.topk_w, R, torch.float32).view(int(T), k),
                    counts=view(v.counts, E, torch.int32),
                    offsets=view(v.offsets, E + 1, torch.int32),
                    perm=view(v.perm, R, torch.int32),
                    inv_perm=view(v.inv_perm, R, torch.int32))

    def set_stage_timing(self, max_forwards: int) -> None:
        _lib.check(self.lib.moe_set_stage_timing(self.handle, int(max_forwards)))

    def stage_times(self):
        """(summed ms per stage as a dict, number of forwards) since the last call."""
        ms = (ctypes.c_float * _lib.MOE_NUM_STAGES)()
        n = ctypes.c_int32()
        _lib.check(self.lib.moe_stage_times(self.handle, ms, _lib.MOE_NUM_STAGES, ctypes.byref(n)))
        return dict(zip(_lib.STAGE_NAMES, [float(v) for v in ms])), int(n.value)

    def expert_bytes(self) -> int:
        """Bytes of one expert's weights (one pool slot) in this layer's format."""
        n = ctypes.c_uint64()
        _lib.check(self.lib.moe_expert_bytes(self.handle, ctypes.byref(n)))
        return n.value

    def upload_expert(self, pool: DeviceWeights, slot: int, src: "HostExpert", stream=None) -> None:
        """Enqueues the copies of one expert (host buffers) into pool slot `slot`."""
        _lib.check(self.lib.moe_expert_upload(self.handle, ctypes.byref(pool.struct()), int(slot),
                                              ctypes.byref(src.struct()), self._stream(stream)))

    def device_flags(self, workspace, T: int, stream=None) -> int:
        f = ctypes.c_uint32()
        _lib.check(self.lib.moe_device_flags(self.handle, _ptr(workspace), int(T), self._stream(stream),
                                             ctypes.byref(f)))
        return int(f.value)


@dataclasses.dataclass
class HostExpert:
    """One expert's weights in page-locked host memory (the pool layout with a
    single slot), the source of moe_expert_upload."""
    tensors: dict

    @classmethod
    def from_pool(cls, weights, expert_slot: int) -> "HostExpert":
        torch = _torch()
        src = weights if isinstance(weights, dict) else {f: getattr(weights, f) for f in WEIGHT_FIELDS}
        out = {}
        for f in WEIGHT_FIELDS:
            a = np.ascontiguousarray(src[f][expert_slot])
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            t = torch.empty(a.shape, dtype=torch.from_numpy(a[:0]).dtype, pin_memory=True)
            t.copy_(torch.from_numpy(a))
            out[f] = t
        return cls(out)

    def struct(self) -> _lib.MoeWeights:
        return _lib.MoeWeights(**{f: _ptr(self.tensors[f]) for f in WEIGHT_FIELDS})


class ExpertCache:
    """The library's set-associative LRU cache of (layer, expert) over pool slots."""

    @staticmethod
    def geometry(free_bytes: int, expert_bytes: int, ways: int):
        """(slots, sets) that fit `free_bytes` for experts of `expert_bytes`."""
        lib = _lib.load()
        s, n = ctypes.c_int32(), ctypes.c_int32()
        _lib.check(lib.moe_cache_geometry(int(free_bytes), int(expert_bytes), int(ways), ctypes.byref(s),
                                          ctypes.byref(n)))
        return s.value, n.value

    def __init__(self, num_sets: int, ways: int, num_experts: int):
        self.lib = _lib.load()
        self.num_experts = num_experts
        h = ctypes.c_void_p()
        _lib.check(self.lib.moe_cache_create(int(num_sets), int(ways), int(num_experts), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.moe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def request(self, layer: int, experts):
        """(slots of `experts`, [(expert, slot) to load], slot table of the layer)."""
        ex = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        n = int(ex.size)
        slots = np.zeros(max(n, 1), np.int32)
        le = np.zeros(max(n, 1), np.int32)
        ls = np.zeros(max(n, 1), np.int32)
        table = np.zeros(self.num_experts, np.int32)
        nl = ctypes.c_int32()
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
        _lib.check(self.lib.moe_cache_request(self.handle, int(layer), p(ex), n, p(slots), p(le), p(ls),
                                              ctypes.byref(nl), p(table)))
        return ([int(v) for v in slots[:n]], [(int(le[i]), int(ls[i])) for i in range(nl.value)],
                [int(v) for v in table])

    def stats(self):
        h, m = ctypes.c_int64(), ctypes.c_int64()
        _lib.check(self.lib.moe_cache_stats(self.handle, ctypes.byref(h), ctypes.byref(m)))
        return int(h.value), int(m.value)
