"""The MoE FFN layer forward, evaluated plainly on the CPU.

Steps, in the order the Strata page describes one decode step:
  1. route every token (section 1.1; router in full precision per the
     Co-inference page, section 5.1);
  2. regroup the routed rows by expert id (section 4.2);
  3. for each expert with rows, look its weights up in the pool slot the
     expert-to-slot table names (the cache slots of the Co-inference page,
     section 2.2), dequantise them (section 3.1) and run the SwiGLU FFN on the
     expert's rows as one matrix product (section 3.2);
  4. scatter the rows back, weighting each token's k expert outputs by its
     gate weights.

precision="f64": every product and sum in fp64 (the reference for tiny
layers).  precision="f32": the dequantised weights (exact in fp32) and the
activations go through fp32 BLAS; routing and the final weighting stay fp64.

A slot id outside [0, num_slots) makes that expert contribute zero (the HIP
path reports such an id through its device error flag).

Shared experts (Strata page, section 2.1: the shared expert common in MoE
models stays resident next to the routed ones).  Reading: a shared expert is
applied to every token with weight exactly 1 and added after the routed
experts; shared expert s is numbered E + s, its weights sit in pool slot
slot_table[E + s], and in the routing it is one more column per token
(topk_idx[t, k + s] = E + s, topk_w[t, k + s] = 1), so the regroup gives it a
group of all T tokens in token order.
"""

import numpy as np

from .codec import dequantize
from .numerics import bf16_to_f64
from .regroup import regroup
from .routing import route


def _silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X, slot, w_gate, w_up, w_down, s_gate, z_gate, s_up, z_up, s_down, z_down, dtype=np.float64,
               bits=4, group=0):
    """Y = Wd (silu(X Wg^T) * (X Wu^T))^T-rows for the rows X [n, d] of one expert."""
    X = np.asarray(X, dtype=dtype)
    Wg = dequantize(w_gate[slot], s_gate[slot], z_gate[slot], dtype, bits, group)
    G = X @ Wg.T
    del Wg
    Wu = dequantize(w_up[slot], s_up[slot], z_up[slot], dtype, bits, group)
    U = X @ Wu.T
    del Wu
    H = _silu(G) * U
    del G, U
    Wd = dequantize(w_down[slot], s_down[slot], z_down[slot], dtype, bits, group)
    return H @ Wd.T


def forward(hidden, router_w, router_b, slot_table, w_gate, w_up, w_down,
            s_gate, z_gate, s_up, z_up, s_down, z_down, top_k, precision="f64", tokens=None,
            num_shared=0, bits=4, group=0):
    """Returns a dict with the routing, the regrouping and out (fp64).

    tokens: optional sorted array of token indices; out then holds only those
    rows (routing and regrouping still cover every token).
    num_shared: shared experts after the E routed ones; slot_table then has
    E + num_shared entries and topk_idx / topk_w have top_k + num_shared
    columns.
    bits, group: the weight format (codec.dequantize): 4 or 8-bit codes, one
    (s, z) per output row (group 0) or per output row and group of K inputs.
    """
    dtype = {"f64": np.float64, "f32": np.float32}[precision]
    hidden = np.asarray(hidden)
    T, d = hidden.shape
    k = int(top_k)
    E = np.asarray(router_w).shape[0]
    S = np.asarray(w_gate).shape[0]
    logits, idx, w = route(hidden, router_w, router_b, k)
    ns = int(num_shared)
    if ns < 0 or np.asarray(slot_table).shape[0] != E + ns:
        raise ValueError("need num_shared >= 0 and E + num_shared slot-table entries")
    if ns:
        idx = np.concatenate([idx, np.broadcast_to(np.arange(E, E + ns, dtype=idx.dtype), (T, ns))], axis=1)
        w = np.concatenate([w, np.ones((T, ns))], axis=1)
        k, E = k + ns, E + ns
    counts, offsets, perm, inv = regroup(idx, E)

    tok_sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    want = np.zeros(T, dtype=bool)
    want[tok_sel] = True

    x = bf16_to_f64(hidden)
    Y = {}  # assignment a -> row of expert output
    wts = dict(w_gate=w_gate, w_up=w_up, w_down=w_down, s_gate=s_gate, z_gate=z_gate,
               s_up=s_up, z_up=z_up, s_down=s_down, z_down=z_down)
    grp = int(group)
    for e in range(E):
        group = perm[offsets[e]:offsets[e + 1]]          # assignments of expert e, ascending
        group = group[want[group // k]]
        if group.size == 0:
            continue
        slot = int(slot_table[e])
        if 0 <= slot < S:
            Ye = expert_ffn(x[group // k], slot, dtype=dtype, bits=bits, group=grp, **wts).astype(np.float64)
        else:
            Ye = np.zeros((group.size, d), dtype=np.float64)
        for r, a in enumerate(group):
            Y[int(a)] = Ye[r]

    out = np.zeros((tok_sel.size, d), dtype=np.float64)
    for i, t in enumerate(tok_sel):
        for j in range(k):
            out[i] += w[t, j] * Y[int(t) * k + j]
    return dict(logits=logits, topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                perm=perm, inv=inv, out=out)
