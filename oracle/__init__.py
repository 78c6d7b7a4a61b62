"""Plain CPU oracle for one Mixture-of-Experts FFN layer forward.

TEST INFRASTRUCTURE.  Only the tests, the smoke entry point and the
benchmark's CPU-baseline leg may import or call anything in this package.  It
shares no code with the HIP path (no kernels, helpers, tables or constants)
and never imports it; the product path must not route through it.

What it computes (the plain definition the regroup -> group GEMM -> combine
route evaluates faster):

    out[t] = sum over the k selected experts e of w[t,e] * FFN_e(x[t])
    FFN_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x)),   silu(z) = z / (1 + exp(-z))
    W_hat    = (q - z) * s       per output row (or per output row and group of
                                 128 inputs), codes q in [0, 15] (int4) or
                                 [0, 255] (8-bit)

with the weights of expert e read from pool slot slot_table[e].  Shared
experts E .. E + S - 1 (if any) are added for every token with weight 1:

    out[t] += sum over s < S of FFN_{E+s}(x[t])

Sources (page titles abbreviated; the pages are the three web pages on
expert offloading for MoE inference):
  * Strata page ("125B MoE at 100+ tok/s on an RTX 3090"):
      section 1.1 -- the router picks the top-2 (or top-1) experts per token;
      section 2.1 -- the shared expert stays resident next to the routed ones;
      section 3.1 -- per-expert int4 with its own scale and zero-point,
                     dequantised to 16-bit before the matrix cores;
      section 3.2 -- the expert FFN is a two-layer MLP, evaluated as a group
                     GEMM over tokens concatenated per expert;
      section 4.2 -- tokens are regrouped by expert id each step.
  * Co-inference page, section 5.1 -- the router stays in full precision;
      8-bit expert weights and grouped quantisation.
  * Mira page, section 4.2 -- Top-K gating.

Readings where the pages are silent (each is listed in the design notes):
selection on fp64 logits with ties to the lower expert id; weights are the
softmax over the k selected logits (equal to softmax-then-renormalise);
SwiGLU experts without biases; stable regroup in expert-id order; a shared
expert is one more expert every token takes with weight exactly 1, after its
routed ones.

Parity pins (tests marked "not gpu"): hand-worked closed forms, W_r = 0 and
k = E special cases, brute-force routing and regrouping by pure-Python loops,
a dense all-experts-then-mask evaluation, a dense SwiGLU via torch's CPU silu,
codec round trips and error bounds, q == z giving exactly zero, exact
power-of-two scale laws, slot-permutation invariance and fp32/fp64 agreement;
for the other weight formats, hand-worked 8-bit and grouped dequantisation,
the reductions grouped-with-row-parameters == per-row and 8-bit with 16x the
int4 codes == int4, and the outlier confinement grouping exists for.
"""

from .numerics import bf16_to_f64, fp16_to_f64  # noqa: F401
from .codec import dequantize, encode_with, pack_codes, quantize, unpack_codes  # noqa: F401
from .routing import router_logits, select_topk, topk_weights, route  # noqa: F401
from .regroup import regroup  # noqa: F401
from .forward import expert_ffn, forward  # noqa: F401
from .brute import brute_dense  # noqa: F401
