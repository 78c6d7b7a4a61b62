"""Dense evaluation: every expert on every token, then mask.

This takes no regrouping at all: it computes FFN_e(x) for all tokens and all
experts and keeps w[t,e] only where e is among token t's k choices.  In exact
arithmetic it equals the regrouped forward, so it pins the regroup, the
per-expert row gathering and the weighted scatter-back independently of how
those are done.  Shared experts (numbered E + s, slot slot_table[E + s]) are
added for every token with weight 1.  Only for tiny layers.
"""

import numpy as np

from .forward import expert_ffn
from .numerics import bf16_to_f64
from .routing import route


def brute_dense(hidden, router_w, router_b, slot_table, w_gate, w_up, w_down,
                s_gate, z_gate, s_up, z_up, s_down, z_down, top_k, num_shared=0, bits=4, group=0):
    x = bf16_to_f64(hidden)
    T, d = x.shape
    E = np.asarray(router_w).shape[0]
    S = np.asarray(w_gate).shape[0]
    _, idx, w = route(hidden, router_w, router_b, int(top_k))
    mask = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(int(top_k)):
            mask[t, idx[t, j]] = w[t, j]
    wts = dict(w_gate=w_gate, w_up=w_up, w_down=w_down, s_gate=s_gate, z_gate=z_gate,
               s_up=s_up, z_up=z_up, s_down=s_down, z_down=z_down)
    out = np.zeros((T, d), dtype=np.float64)
    for e in range(E):
        slot = int(slot_table[e])
        if not 0 <= slot < S:
            continue
        F = expert_ffn(x, slot, dtype=np.float64, bits=bits, group=group, **wts)
        out += mask[:, e:e + 1] * F
    for e in range(E, E + int(num_shared)):   # shared experts: every token, weight 1
        slot = int(slot_table[e])
        if 0 <= slot < S:
            out += expert_ffn(x, slot, dtype=np.float64, bits=bits, group=group, **wts)
    return out
