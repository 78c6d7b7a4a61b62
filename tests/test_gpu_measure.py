"""The read-stream yardstick bench.py reports next to the layer: it must read
every byte it is given (its XOR fold equals the buffer's) for any grid."""

import numpy as np
import pytest

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096, 3), ((1 << 20) + 48, 7), (64 << 20, 2048)])
def test_read_probe_reads_every_word(nbytes, blocks):
    torch = require_gpu()
    from expert_ffn_layer_router_amd import hbm_read_probe
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"read probe: {nbytes} bytes, {blocks} blocks")
    hbm_read_probe(buf, sink, blocks)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(host)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == expect
