"""moe_forward_noalloc (the forward on the library's own device scratch, for
callers that cannot allocate) against moe_forward with a caller workspace:
the same kernels, so the outputs must agree bit for bit, which is tighter than
the 2e-2 bar the oracle parity tests use.  Two calls in a row, the second with
fewer tokens, so that the second reads a scratch the first left behind."""

import numpy as np
import pytest

import synth
from gpu_util import GpuLayer, require_gpu, say

pytestmark = pytest.mark.gpu


def _bits(out):
    torch = require_gpu()
    return out.detach().cpu().view(torch.int16).numpy().copy()


@pytest.mark.parametrize("name,Ts", [("fine_tiny", (48, 7)), ("tiny_q8g128", (64, 5)),
                                     ("mixtral_decode", (16, 3)), ("phi35_skew", (64, 33))])
def test_noalloc_matches_workspace_forward(name, Ts):
    torch = require_gpu()
    case = synth.make_case(name, T=max(Ts))
    g = GpuLayer(case.shape, case.weights, max_tokens=max(Ts))
    d = case.shape.d_model
    for T in Ts:
        x = g.hidden(synth.make_hidden(T, d, seed=T))
        ref = g.layer.forward(x, g.router_w, g.router_b, g.slot_table, g.dw)
        out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        say(f"{name}: noalloc forward, T={T}")
        g.layer.forward_noalloc(x, g.router_w, g.router_b, g.slot_table, g.dw, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(out), _bits(ref), err_msg=f"{name} T={T}")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    torch = require_gpu()
    from expert_ffn_layer_router_amd import MoeError
    from expert_ffn_layer_router_amd import _lib
    case = synth.make_case("tiny", T=65536)
    g = GpuLayer(case.shape, case.weights, max_tokens=65536)
    x = g.hidden(case.hidden)
    out = torch.zeros((65536, case.shape.d_model), dtype=torch.bfloat16, device="cuda")
    assert g.layer.workspace_size(65536) > 16 << 20
    say("tiny: noalloc with T=65536 must be refused")
    with pytest.raises(MoeError) as ei:
        g.layer.forward_noalloc(x, g.router_w, g.router_b, g.slot_table, g.dw, out)
    assert ei.value.status == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).abs().sum().item()) == 0     # nothing was enqueued
