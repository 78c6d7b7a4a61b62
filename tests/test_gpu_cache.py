"""Slot-pool refill on the GPU: a pool of fewer slots than (layer, expert)
pairs, managed by the library's expert cache.  Each step and layer, the
forward runs with the cache's slot table; when a routed expert is missing
(the device flag), the routed experts are requested from the cache, the
loads are copied from page-locked host memory on a second stream, the compute
stream waits for them, and the forward runs again -- and must match the
oracle.  Co-inference page, sections 2.2 and 3.1; Strata page, section 2.2."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits_to_f64, require_gpu, say
from conftest import assert_out_close, weights_kwargs
from test_gpu_parity import check_routing

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,group", [(4, 0), (8, 128)])
def test_refill_from_host_on_a_copy_stream_matches_the_oracle(bits, group):
    torch = require_gpu()
    from expert_ffn_layer_router_amd import (DeviceWeights, ExpertCache, HostExpert, MOE_FLAG_BAD_SLOT, MoeLayer,
                                             to_device)
    L, T = 3, 2
    shape = synth.LayerShape(T, 128, 256, 8, 2, 8, "identity", 0.0, 0, bits, group)
    layers = [synth.make_weights(shape, seed=10 + i) for i in range(L)]
    host = [[HostExpert.from_pool(w, e) for e in range(shape.num_experts)] for w in layers]
    pool = DeviceWeights.upload(layers[0])          # 8 slots; their first contents are never used
    cache = ExpertCache(num_sets=2, ways=4, num_experts=shape.num_experts)   # layers 0 and 2 share set 0
    g = MoeLayer(shape.d_model, shape.d_ff, shape.num_experts, shape.top_k, shape.num_slots, T,
                 weight_bits=bits, group_size=group)
    ws = g.new_workspace(T)
    out = torch.empty((T, shape.d_model), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()  # the zero fill and the pool upload run on the default stream
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    rws = [to_device(w.router_w) for w in layers]
    table = [cache.request(i, [])[2] for i in range(L)]
    reruns = 0
    for step in range(5):
        x_bits = synth.make_hidden(T, shape.d_model, seed=100 + step)
        x = to_device(x_bits).view(torch.bfloat16)
        for i in range(L):
            say(f"refill: step {step} layer {i}")
            st = to_device(np.asarray(table[i], np.int32))
            g.forward(x, rws[i], None, st, pool, out=out, workspace=ws, stream=compute)
            compute.synchronize()
            if g.device_flags(ws, T, stream=compute) & MOE_FLAG_BAD_SLOT:
                routed = g.routing(ws, T)["topk_idx"].cpu().numpy().ravel().tolist()
                slots, loads, table[i] = cache.request(i, routed)
                for e, slot in loads:
                    g.upload_expert(pool, slot, host[i][e], stream=copy)
                ev = torch.cuda.Event()
                ev.record(copy)
                compute.wait_event(ev)
                st = to_device(np.asarray(table[i], np.int32))
                g.forward(x, rws[i], None, st, pool, out=out, workspace=ws, stream=compute)
                compute.synchronize()
                assert g.device_flags(ws, T, stream=compute) == 0
                reruns += 1
            res = {k: v.cpu().numpy() for k, v in g.routing(ws, T).items()}
            ref = oracle.forward(x_bits, top_k=shape.top_k, precision="f64", bits=bits, group=group,
                                 **weights_kwargs(layers[i]))
            check_routing(res, ref)
            assert_out_close(bf16_bits_to_f64(out), ref["out"])
    hits, misses = cache.stats()
    say(f"refill: {reruns} reruns, cache hits {hits}, misses {misses}")
    assert misses > 0 and hits > 0 and reruns > 0
