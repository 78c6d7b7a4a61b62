"""MI355X (gfx950) Mixture-of-Experts FFN layer forward.

The layer (router top-k, regroup by expert, int4 grouped GEMM with SwiGLU,
weighted scatter-back) runs in hand-written HIP kernels behind the C ABI of
include/moe.h; this package is its thin Python binding.
"""

from ._lib import MoeError, load, MOE_FLAG_BAD_SLOT  # noqa: F401
from .layer import DeviceWeights, ExpertCache, HostExpert, MoeLayer, hbm_read_probe, to_device  # noqa: F401
