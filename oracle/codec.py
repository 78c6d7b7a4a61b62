"""Per-expert asymmetric integer codecs: int4 or 8-bit codes, one scale and
zero-point per output row or per (output row, group of K inputs).

Strata page, section 3.1: each expert is quantised on its own, with its own
scale and zero-point; the weights are stored as packed int4 and turned back
into 16-bit values before the matrix multiply.  Co-inference page, section
5.1: 8-bit expert weights are a further option, the router stays in full
precision, and grouped quantisation keeps the precision loss down (a weight
outlier then only widens the range of its own group).

Readings taken for the details the pages leave open:
  * unsigned codes 0 .. 2^bits - 1; int4 codes two per byte along K with the
    even k in the low nibble, 8-bit codes one per byte;
  * scale s in fp16 and an integer zero-point z held as fp16;
  * group == 0: one (s, z) per output row, arrays [N];
    group == G > 0: one (s, z) per output row and run of G consecutive k,
    arrays [K/G, N] (group-major: row g holds group g of every output row);
  * dequantisation is W_hat = (q - z) * s.
"""

import numpy as np

from .numerics import fp16_to_f64


def unpack_codes(packed: np.ndarray, bits: int = 4) -> np.ndarray:
    """Bytes -> codes.  bits 4: [..., K/2] -> [..., K], byte m holding k = 2m
    (low nibble) and 2m+1 (high); bits 8: one code per byte."""
    p = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return p.copy()
    if bits != 4:
        raise ValueError("bits must be 4 or 8")
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    q[..., 0::2] = p & 0x0F
    q[..., 1::2] = p >> 4
    return q


def pack_codes(q: np.ndarray, bits: int = 4) -> np.ndarray:
    """Codes in 0 .. 2^bits - 1 -> bytes (inverse of unpack_codes)."""
    q = np.asarray(q, dtype=np.uint8)
    if bits == 8:
        return q.copy()
    if bits != 4:
        raise ValueError("bits must be 4 or 8")
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    if q.size and q.max() > 15:
        raise ValueError("codes must lie in 0..15")
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def _per_element(v: np.ndarray, K: int, group: int) -> np.ndarray:
    """Scale or zero-point arrays -> one value per weight [N, K]."""
    if group == 0:
        return v[..., :, None]
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    if v.shape[-2] != K // group:
        raise ValueError("grouped parameters must have K/group rows")
    return np.repeat(np.swapaxes(v, -1, -2), group, axis=-1)


def dequantize(packed: np.ndarray, s_bits: np.ndarray, z_bits: np.ndarray, dtype=np.float64, bits: int = 4,
               group: int = 0) -> np.ndarray:
    """W_hat[n, k] = (q[n, k] - z) * s with the (s, z) of row n (group 0) or of
    row n and group k // group.

    With integer z the product has at most 8 + 11 significant bits, so it is
    exact in fp32 as well as fp64; a non-integer z is handled by the same
    formula.
    """
    q = unpack_codes(packed, bits).astype(dtype)
    K = q.shape[-1]
    s = _per_element(fp16_to_f64(s_bits).astype(dtype), K, group)
    z = _per_element(fp16_to_f64(z_bits).astype(dtype), K, group)
    q -= z
    q *= s
    return q


def _row_params(seg: np.ndarray, qmax: int):
    """(s fp16, z) of one run of weights: its range widened to include 0."""
    lo = min(np.float32(seg.min()), np.float32(0.0))
    hi = max(np.float32(seg.max()), np.float32(0.0))
    s16 = np.float16(np.float32(hi - lo) / np.float32(qmax))
    if s16 == 0:
        s16 = np.float16(1.0)
    z = np.float32(min(max(np.rint(np.float32(-lo) / np.float32(s16)), 0.0), float(qmax)))
    return s16, np.float16(z)


def quantize(W: np.ndarray, bits: int = 4, group: int = 0):
    """Encode fp32 rows: returns (packed codes, scale fp16 bits, zero fp16 bits).

    Per row (group 0) or per (row, group): the range [lo, hi] is widened to
    include 0; s = fp16((hi-lo)/qmax), replaced by 1 when it rounds to 0;
    z = clip(rint(-lo/s), 0, qmax); q = clip(rint(W/s) + z, 0, qmax), with
    qmax = 2^bits - 1.  Arithmetic in fp32, rint ties to even.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    qmax = (1 << bits) - 1
    G = K if group == 0 else group
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    ng = K // G
    s_out = np.empty((ng, N), dtype=np.float16)
    z_out = np.empty((ng, N), dtype=np.float16)
    q_out = np.empty(W.shape, dtype=np.uint8)
    for n in range(N):
        for g in range(ng):
            seg = W[n, g * G:(g + 1) * G]
            s16, z16 = _row_params(seg, qmax)
            s_out[g, n], z_out[g, n] = s16, z16
            q = np.rint(seg / np.float32(s16)) + np.float32(z16)
            q_out[n, g * G:(g + 1) * G] = np.clip(q, 0, qmax).astype(np.uint8)
    if group == 0:
        s_out, z_out = s_out[0], z_out[0]
    return pack_codes(q_out, bits), s_out.view(np.uint16), z_out.view(np.uint16)


def encode_with(W: np.ndarray, s_bits: np.ndarray, z_bits: np.ndarray, bits: int = 4, group: int = 0) -> np.ndarray:
    """Codes of W for given (s, z): clip(rint(W/s) + z, 0, 2^bits - 1), fp32."""
    W = np.asarray(W, dtype=np.float32)
    K = W.shape[-1]
    s = _per_element(np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.float16).astype(np.float32), K, group)
    z = _per_element(np.ascontiguousarray(z_bits, dtype=np.uint16).view(np.float16).astype(np.float32), K, group)
    q = np.rint(W / s) + z
    return np.clip(q, 0, (1 << bits) - 1).astype(np.uint8)
