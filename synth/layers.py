"""Seeded synthetic MoE layers shaped like the workloads the pages discuss.

Shapes: a tiny layer, Mixtral-8x7B-like experts (d=4096, d_ff=14336, 8 experts,
top-2; the Co-inference page, section 2.2, sizes one such fp16 expert at 340 MB),
Phi-3.5-MoE-like experts (d_ff=6400, 16 experts; 152 MB per fp16 expert in the
same page, section 4.1) and a fine-grained 64-expert top-6 layer.  The Strata
page (section 4.2 and 5.3) fixes the batch-16 decode step and the 2048-token
prefill chunk.

Recipe (all streams are independent PCG64 generators keyed by (seed, tag, i),
so a layer's weights do not depend on the token count and matrices can be drawn
in parallel):
  * hidden  ~ N(0,1) drawn in fp32, rounded to bf16 (round to nearest even);
  * router  W_r ~ N(0,1)/sqrt(d) in fp32; optional bias b_e = -s * ln(e+1),
    a log-Zipf(s) preference for low expert ids (expert 0 hottest);
  * experts W_gate, W_up ~ N(0,1)/sqrt(d) of shape [d_ff, d] and
    W_down ~ N(0,1)/sqrt(d_ff) of shape [d, d_ff], each encoded to asymmetric
    unsigned int4 with one fp16 scale and one integer zero-point (stored as
    fp16) per output row -- the per-expert quantisation of the Strata page,
    section 3.1 -- or, for the other weight formats, to 8-bit codes and/or
    one (s, z) per output row and group of 128 inputs (the 8-bit, grouped
    quantisation of the Co-inference page, section 5.1);
  * shared experts (num_shared > 0) are drawn like routed experts E, E+1, ...
    and have no router row;
  * the pool has num_slots slots; expert e lives at slot slot_table[e];
    slots no expert uses are filled with random codes and NaN scales so that a
    wrong indirection cannot go unnoticed.

Encoding rule (input preparation, not part of the layer's forward): per row
(or per row and group), lo = min(min W, 0), hi = max(max W, 0),
s = fp16((hi-lo)/qmax) (1 if that is 0), z = clip(rint(-lo/s), 0, qmax),
q = clip(rint(W/s) + z, 0, qmax), qmax = 2^bits - 1, all in fp32 with
round-half-to-even; int4: two codes per byte along K, low nibble = even k;
grouped parameters are stored group-major, [K/G][N].
"""

from __future__ import annotations

import dataclasses
import json
import os
import tempfile
from concurrent.futures import ThreadPoolExecutor
from functools import lru_cache
from typing import Optional

import numpy as np

# stream tags
_HIDDEN, _ROUTER, _GATE, _UP, _DOWN, _SLOTS, _POISON = 1, 2, 3, 4, 5, 6, 7
_FP16_NAN = np.uint16(0x7E00)
_CACHE_VERSION = 1


@dataclasses.dataclass(frozen=True)
class LayerShape:
    T: int
    d_model: int
    d_ff: int
    num_experts: int
    top_k: int
    num_slots: int
    slot_kind: str = "identity"   # identity | perm (all slots, shuffled) | sparse (E + shared of S slots)
    zipf_s: float = 0.0           # 0: no router bias
    num_shared: int = 0           # shared experts (every token, weight 1), numbered E .. E + num_shared - 1
    bits: int = 4                 # code width: 4 or 8
    group: int = 0                # 0: one (s, z) per output row; G: per output row and run of G inputs

    def family(self) -> tuple:
        """Everything but T and top_k: layers that differ only in those share weights."""
        return (self.d_model, self.d_ff, self.num_experts, self.num_slots,
                self.slot_kind, float(self.zipf_s), int(self.num_shared), int(self.bits), int(self.group))


CASES = {
    # tiny layer, seconds on a CPU
    "tiny": LayerShape(16, 128, 256, 8, 2, 8, "identity", 0.0),
    # Mixtral-8x7B-shaped layer: batch-16 decode step and a 2048-token prefill chunk
    "mixtral_decode": LayerShape(16, 4096, 14336, 8, 2, 8, "identity", 0.0),
    "mixtral_prefill": LayerShape(2048, 4096, 14336, 8, 2, 8, "identity", 0.0),
    # Phi-3.5-MoE-shaped layer, Zipf(1.2)-skewed routing, shuffled 16-slot pool
    "phi35_skew": LayerShape(64, 4096, 6400, 16, 2, 16, "perm", 1.2),
    # fine-grained 64-expert top-6 layer living in a 128-slot pool
    "fine_decode": LayerShape(16, 4096, 2048, 64, 6, 128, "sparse", 1.0),
    "fine_prefill": LayerShape(4096, 4096, 2048, 64, 6, 128, "sparse", 1.0),
    # the fine-grained routing structure at tiny width (CPU brute force)
    "fine_tiny": LayerShape(16, 128, 256, 64, 6, 128, "sparse", 1.0),
    # top-1 routing plus one shared expert of the same shape (Mixtral-8x7B-shaped
    # experts): a batch-16 decode step and a 2048-token prefill chunk
    "shared_decode": LayerShape(16, 4096, 14336, 8, 1, 9, "identity", 0.0, 1),
    "shared_prefill": LayerShape(2048, 4096, 14336, 8, 1, 9, "identity", 0.0, 1),
    # the same structure at tiny width, and fine-grained top-6 with two shared
    # experts (8 experts per token), both with scattered slots
    "shared_tiny": LayerShape(16, 128, 256, 8, 1, 12, "sparse", 1.0, 1),
    "fine_shared_tiny": LayerShape(16, 128, 256, 64, 6, 80, "sparse", 1.0, 2),
    # other weight formats: int4 with (s, z) per output row and group of 128
    # inputs, and 8-bit codes per row or per group of 128
    "mixtral_decode_q4g128": LayerShape(16, 4096, 14336, 8, 2, 8, "identity", 0.0, 0, 4, 128),
    "mixtral_prefill_q4g128": LayerShape(2048, 4096, 14336, 8, 2, 8, "identity", 0.0, 0, 4, 128),
    "mixtral_decode_q8g128": LayerShape(16, 4096, 14336, 8, 2, 8, "identity", 0.0, 0, 8, 128),
    "mixtral_prefill_q8g128": LayerShape(2048, 4096, 14336, 8, 2, 8, "identity", 0.0, 0, 8, 128),
    "phi35_skew_q8": LayerShape(64, 4096, 6400, 16, 2, 16, "perm", 1.2, 0, 8, 0),
    # tiny widths with several groups along both K (d = 256, d_ff = 384: the
    # down K is not a multiple of 256)
    "tiny_q4g128": LayerShape(16, 256, 384, 8, 2, 12, "sparse", 1.0, 0, 4, 128),
    "tiny_q8": LayerShape(16, 256, 384, 8, 2, 12, "sparse", 1.0, 0, 8, 0),
    "tiny_q8g128": LayerShape(16, 256, 384, 8, 2, 12, "sparse", 1.0, 1, 8, 128),
}


def case_shape(name: str, T: Optional[int] = None) -> LayerShape:
    shp = CASES[name]
    return shp if T is None else dataclasses.replace(shp, T=int(T))


@dataclasses.dataclass
class Weights:
    """One layer's weights, pool-indexed by slot.  Half-precision arrays hold
    IEEE fp16 bit patterns (uint16)."""
    router_w: np.ndarray            # fp32 [E, d] (routed experts only)
    router_b: Optional[np.ndarray]  # fp32 [E] or None
    slot_table: np.ndarray          # int32 [E + num_shared]
    w_gate: np.ndarray              # uint8 [S, d_ff, d/2]
    w_up: np.ndarray                # uint8 [S, d_ff, d/2]
    w_down: np.ndarray              # uint8 [S, d, d_ff/2]
    s_gate: np.ndarray              # uint16 [S, d_ff]
    z_gate: np.ndarray
    s_up: np.ndarray
    z_up: np.ndarray
    s_down: np.ndarray              # uint16 [S, d]
    z_down: np.ndarray

    ARRAYS = ("router_w", "router_b", "slot_table", "w_gate", "w_up", "w_down",
              "s_gate", "z_gate", "s_up", "z_up", "s_down", "z_down")

    def nbytes(self) -> int:
        return sum(getattr(self, a).nbytes for a in self.ARRAYS if getattr(self, a) is not None)


@dataclasses.dataclass
class Case:
    name: str
    shape: LayerShape
    seed: int
    hidden: np.ndarray              # uint16 bf16 bits [T, d]
    weights: Weights


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag, index))))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _encode_rows(W: np.ndarray, bits: int = 4, group: int = 0):
    """Asymmetric per-row (group 0) or per-(row, group) integer encoding of an
    fp32 matrix (input preparation).  Returns (codes as stored, s bits, z bits),
    the parameters [N] or [K/group, N]."""
    N, K = W.shape
    qmax = np.float32((1 << bits) - 1)
    G = K if group == 0 else group
    Wg = W.reshape(N, K // G, G)
    lo = np.minimum(Wg.min(axis=2), np.float32(0))
    hi = np.maximum(Wg.max(axis=2), np.float32(0))
    s16 = ((hi - lo) / qmax).astype(np.float16)
    s16[s16 == 0] = np.float16(1)
    s = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / s), 0, qmax).astype(np.float32)
    q = Wg / s[:, :, None]
    np.rint(q, out=q)
    q += z[:, :, None]
    np.clip(q, 0, qmax, out=q)
    q8 = q.reshape(N, K).astype(np.uint8)
    del q
    packed = q8 if bits == 8 else (q8[:, 0::2] | (q8[:, 1::2] << 4)).astype(np.uint8)
    s16, z16 = s16.T, z.astype(np.float16).T            # [K/G, N]
    if group == 0:
        s16, z16 = s16[0], z16[0]
    return np.ascontiguousarray(packed), np.ascontiguousarray(s16).view(np.uint16), \
        np.ascontiguousarray(z16).view(np.uint16)


def draw_dense_expert(shape: LayerShape, seed: int, e: int):
    """The fp32 matrices (before encoding) of expert e: (W_gate, W_up, W_down)."""
    d, f = shape.d_model, shape.d_ff
    wg = _rng(seed, _GATE, e).standard_normal((f, d), dtype=np.float32) * np.float32(1 / np.sqrt(d))
    wu = _rng(seed, _UP, e).standard_normal((f, d), dtype=np.float32) * np.float32(1 / np.sqrt(d))
    wd = _rng(seed, _DOWN, e).standard_normal((d, f), dtype=np.float32) * np.float32(1 / np.sqrt(f))
    return wg, wu, wd


def _draw_matrix(seed, tag, e, rows, cols, fan_in, bits=4, group=0):
    W = _rng(seed, tag, e).standard_normal((rows, cols), dtype=np.float32)
    W *= np.float32(1 / np.sqrt(fan_in))
    return _encode_rows(W, bits, group)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cache_dir() -> str:
    return os.environ.get("MOE_SYNTH_CACHE") or os.path.join(tempfile.gettempdir(), "moe_synth_cache")


def _cache_key(shape: LayerShape, seed: int) -> str:
    d, f, E, S, kind, zs, ns, bits, group = shape.family()
    shared = f"_sh{ns}" if ns else ""
    fmt = "" if (bits, group) == (4, 0) else f"_b{bits}g{group}"
    return f"v{_CACHE_VERSION}_d{d}_f{f}_E{E}{shared}_S{S}_{kind}_z{zs:g}{fmt}_seed{seed}"


def _load_cached(key: str) -> Optional[Weights]:
    path = os.path.join(_cache_dir(), key)
    if not os.path.isfile(os.path.join(path, "done.json")):
        return None
    arrs = {}
    for a in Weights.ARRAYS:
        p = os.path.join(path, a + ".npy")
        arrs[a] = np.load(p, allow_pickle=False) if os.path.exists(p) else None
    return Weights(**arrs)


def _store_cached(key: str, w: Weights) -> None:
    root = _cache_dir()
    try:
        os.makedirs(root, exist_ok=True)
        tmp = tempfile.mkdtemp(prefix=key + ".", dir=root)
        for a in Weights.ARRAYS:
            v = getattr(w, a)
            if v is not None:
                np.save(os.path.join(tmp, a + ".npy"), v, allow_pickle=False)
        with open(os.path.join(tmp, "done.json"), "w") as fh:
            json.dump({"key": key}, fh)
        os.replace(tmp, os.path.join(root, key))
    except OSError:
        pass  # the cache is an optimisation only


def _generate_weights(shape: LayerShape, seed: int) -> Weights:
    d, f, S = shape.d_model, shape.d_ff, shape.num_slots
    Er = shape.num_experts                 # routed experts (router rows)
    E = Er + shape.num_shared              # every expert with weights, shared ones last
    if d % 2 or f % 2:
        raise ValueError("d_model and d_ff must be even (two int4 codes per byte)")
    router_w = _rng(seed, _ROUTER).standard_normal((Er, d), dtype=np.float32) * np.float32(1 / np.sqrt(d))
    router_b = None
    if shape.zipf_s:
        router_b = (-float(shape.zipf_s) * np.log(np.arange(1, Er + 1, dtype=np.float64))).astype(np.float32)
    if shape.slot_kind == "identity":
        if S < E:
            raise ValueError("identity slot table needs num_slots >= num_experts")
        slot_table = np.arange(E, dtype=np.int32)
    elif shape.slot_kind == "perm":
        if S != E:
            raise ValueError("perm slot table needs num_slots == num_experts")
        slot_table = _rng(seed, _SLOTS).permutation(S).astype(np.int32)
    elif shape.slot_kind == "sparse":
        if S < E:
            raise ValueError("sparse slot table needs num_slots >= num_experts")
        slot_table = _rng(seed, _SLOTS).permutation(S)[:E].astype(np.int32)
    else:
        raise ValueError(f"unknown slot_kind {shape.slot_kind!r}")

    bits, group = shape.bits, shape.group
    if bits not in (4, 8) or group < 0 or (group and (d % group or f % group)):
        raise ValueError("bits must be 4 or 8 and the group size must divide d_model and d_ff")
    w_gate = np.empty((S, f, d * bits // 8), np.uint8)
    w_up = np.empty((S, f, d * bits // 8), np.uint8)
    w_down = np.empty((S, d, f * bits // 8), np.uint8)
    gu_p = (S, f) if group == 0 else (S, d // group, f)      # scale / zero-point shapes
    dn_p = (S, d) if group == 0 else (S, f // group, d)
    s_gate = np.empty(gu_p, np.uint16); z_gate = np.empty(gu_p, np.uint16)
    s_up = np.empty(gu_p, np.uint16); z_up = np.empty(gu_p, np.uint16)
    s_down = np.empty(dn_p, np.uint16); z_down = np.empty(dn_p, np.uint16)

    jobs = []
    for e in range(E):
        sl = int(slot_table[e])
        jobs.append((_GATE, e, f, d, d, (w_gate, s_gate, z_gate), sl))
        jobs.append((_UP, e, f, d, d, (w_up, s_up, z_up), sl))
        jobs.append((_DOWN, e, d, f, f, (w_down, s_down, z_down), sl))

    def run(job):
        tag, e, rows, cols, fan_in, (wq, ws, wz), sl = job
        p, s, z = _draw_matrix(seed, tag, e, rows, cols, fan_in, bits, group)
        wq[sl], ws[sl], wz[sl] = p, s, z

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))

    used = set(int(s) for s in slot_table)
    for sl in range(S):
        if sl in used:
            continue
        r = _rng(seed, _POISON, sl)
        for wq, ws, wz in ((w_gate, s_gate, z_gate), (w_up, s_up, z_up), (w_down, s_down, z_down)):
            wq[sl] = r.integers(0, 256, size=wq.shape[1:], dtype=np.uint8)
            ws[sl] = _FP16_NAN
            wz[sl] = r.integers(0, 1 << bits, size=wz.shape[1:]).astype(np.float16).view(np.uint16)

    return Weights(router_w=router_w, router_b=router_b, slot_table=slot_table,
                   w_gate=w_gate, w_up=w_up, w_down=w_down, s_gate=s_gate, z_gate=z_gate,
                   s_up=s_up, z_up=z_up, s_down=s_down, z_down=z_down)


@lru_cache(maxsize=2)
def _weights_memo(family: tuple, top_k: int, seed: int) -> Weights:
    shape = LayerShape(0, family[0], family[1], family[2], top_k, family[3], *family[4:])
    big = shape.num_slots * 3 * shape.d_model * shape.d_ff // 2 > (64 << 20)
    key = _cache_key(shape, seed)
    if big:
        w = _load_cached(key)
        if w is not None:
            return w
    w = _generate_weights(shape, seed)
    if big:
        _store_cached(key, w)
    return w


def make_weights(shape: LayerShape, seed: int = 0) -> Weights:
    """Weights of the layer family (shared by every T)."""
    return _weights_memo(shape.family(), 0, int(seed))


def make_hidden(T: int, d_model: int, seed: int = 0) -> np.ndarray:
    x = _rng(seed, _HIDDEN).standard_normal((T, d_model), dtype=np.float32)
    return bf16_bits_from_f32(x)


def make_case(name: str, seed: int = 0, T: Optional[int] = None) -> Case:
    shape = case_shape(name, T)
    return Case(name=name, shape=shape, seed=seed,
                hidden=make_hidden(shape.T, shape.d_model, seed),
                weights=make_weights(shape, seed))
