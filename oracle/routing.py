"""Router: logits, top-k selection and the renormalised gate weights.

Strata page, section 1.1: a router picks the top-2 (or top-1) experts for each
token.  Co-inference page, section 5.1: the router is kept in full precision.
Mira page, section 4.2: Top-K gating.

Readings: logits are l = x W_r^T + b in fp64 (each bf16 x fp32 product is exact
in fp64); the k largest logits are taken in the order (logit descending,
expert id ascending), so ties go to the lower expert id; the gate weights are
the softmax over the selected logits, which equals a softmax over all experts
renormalised over the k selected ones.
"""

import numpy as np

from .numerics import bf16_to_f64


def router_logits(hidden_bits, router_w, router_b=None) -> np.ndarray:
    x = bf16_to_f64(hidden_bits)
    W = np.asarray(router_w, dtype=np.float32).astype(np.float64)
    logits = x @ W.T
    if router_b is not None:
        logits = logits + np.asarray(router_b, dtype=np.float32).astype(np.float64)[None, :]
    return logits


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """topk_idx[t] = the first k experts in the order (-logit, expert id)."""
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -logits), axis=-1)
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(logits, topk_idx.astype(np.int64), axis=1)
    e = np.exp(sel - sel[:, :1])
    return e / e.sum(axis=1, keepdims=True)


def route(hidden_bits, router_w, router_b, k: int):
    """Returns (logits fp64 [T,E], topk_idx int32 [T,k], topk_w fp64 [T,k])."""
    logits = router_logits(hidden_bits, router_w, router_b)
    idx = select_topk(logits, k)
    return logits, idx, topk_weights(logits, idx)
