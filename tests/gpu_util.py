"""Helpers for the GPU tests: run the layer through the C ABI and bring the
results back as numpy arrays."""

import sys

import numpy as np
import pytest


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits_to_f64(t):
    """torch bf16/int16 tensor on any device -> float64 numpy array."""
    a = t.detach().cpu().contiguous().view(dtype=__import__("torch").int16).numpy().view(np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class GpuLayer:
    """A layer shape with its weights resident on the device."""

    def __init__(self, shape, weights, max_tokens=None):
        torch = require_gpu()
        from expert_ffn_layer_router_amd import DeviceWeights, MoeLayer, to_device
        self.torch = torch
        self.shape = shape
        self.weights = weights
        self.layer = MoeLayer(shape.d_model, shape.d_ff, shape.num_experts, shape.top_k, shape.num_slots,
                              max_tokens or max(shape.T, 1), num_shared=shape.num_shared,
                              weight_bits=shape.bits, group_size=shape.group)
        self.dw = DeviceWeights.upload(weights)
        self.router_w = to_device(weights.router_w)
        self.router_b = None if weights.router_b is None else to_device(weights.router_b)
        self.slot_table = to_device(weights.slot_table)
        self.to_device = to_device

    def hidden(self, hidden_bits):
        return self.to_device(hidden_bits).view(self.torch.bfloat16)

    def run(self, hidden_bits, slot_table=None, router_w=None, router_b="same"):
        torch = self.torch
        T = hidden_bits.shape[0]
        x = self.hidden(hidden_bits)
        ws = self.layer.new_workspace(T)
        st = self.slot_table if slot_table is None else self.to_device(np.asarray(slot_table, np.int32))
        rw = self.router_w if router_w is None else self.to_device(np.asarray(router_w, np.float32))
        rb = self.router_b if isinstance(router_b, str) else (
            None if router_b is None else self.to_device(np.asarray(router_b, np.float32)))
        out = self.layer.forward(x, rw, rb, st, self.dw, workspace=ws)
        torch.cuda.synchronize()
        res = {k: v.cpu().numpy() for k, v in self.layer.routing(ws, T).items()}
        res["out"] = bf16_bits_to_f64(out)
        res["out_bits"] = out.detach().cpu().view(torch.int16).numpy().copy()
        res["flags"] = self.layer.device_flags(ws, T)
        return res
