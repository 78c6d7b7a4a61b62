"""GPU parity on a seeded sweep of small layers: random expert counts, top-k,
shared experts, widths (including widths that are not multiples of 256, so
the half-stage and narrow-block paths run), weight formats, token counts on
both sides of the decode / prefill boundary, and scattered slot tables.
Each case is checked against the oracle like the named workloads."""

import random

import numpy as np
import pytest

import synth
from conftest import assert_out_close
from gpu_util import GpuLayer, require_gpu, say
from test_gpu_parity import _oracle, check_routing

pytestmark = pytest.mark.gpu


def _shape(seed):
    r = random.Random(1000 + seed)
    E = r.choice([1, 2, 3, 8, 13, 32, 70])
    k = r.randint(1, min(E, 8))
    ns = r.randint(0, min(8 - k, 2))
    if seed < 24:   # narrow layers
        d = r.choice([128, 256, 384])
        f = r.choice([128, 256, 384, 640])
    else:           # wider ones: the full-width prefill blocks and longer k loops
        d = r.choice([512, 1024, 1152])
        f = r.choice([768, 1024, 1536])
    bits, group = r.choice([(4, 0), (4, 128), (8, 0), (8, 128)])
    T = r.choice([1, 7, 16, 33, 64, 65, 200, 700] if seed < 24 else [5, 16, 48, 64, 130, 1500])
    slots = E + ns + r.randint(0, 8)
    zipf = r.choice([0.0, 1.0, 2.5])
    return synth.LayerShape(T, d, f, E, k, slots, "sparse", zipf, ns, bits, group)


@pytest.mark.parametrize("seed", range(36))
def test_random_layer(seed):
    require_gpu()
    shape = _shape(seed)
    w = synth.make_weights(shape, seed=seed)
    x = synth.make_hidden(shape.T, shape.d_model, seed=seed)
    case = synth.Case(f"sweep{seed}", shape, seed, x, w)
    say(f"sweep {seed}: {shape}")
    res = GpuLayer(shape, w, max_tokens=shape.T).run(x)
    ref = _oracle(case)
    check_routing(res, ref)
    assert res["flags"] == 0
    assert_out_close(res["out"], ref["out"])
