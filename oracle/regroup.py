"""Regroup routed rows by expert id.

Strata page, section 4.2: after routing, all tokens are reordered by the
expert they chose so that each expert's tokens are contiguous and its weights
are loaded once for all of them; section 3.2 then runs one group GEMM over
these contiguous groups.

Reading: assignment a = t*k + j (token t's j-th choice) is a row; rows are
grouped in expert-id order and keep ascending a inside a group (a stable
sort).  perm[p] is the assignment at grouped position p, inv[a] its position.
"""

import numpy as np


def regroup(topk_idx: np.ndarray, num_experts: int):
    """Returns (counts [E], offsets [E+1], perm [R], inv [R]) as int32."""
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    perm = np.argsort(flat, kind="stable")
    inv = np.empty_like(perm)
    inv[perm] = np.arange(flat.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))
