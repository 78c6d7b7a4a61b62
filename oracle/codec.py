"""Per-expert asymmetric int4 codec.

Strata page, section 3.1: each expert is quantised on its own, with its own
scale and zero-point; the weights are stored as packed int4 and turned back
into 16-bit values before the matrix multiply.  Reading taken for the details
the page leaves open: unsigned codes 0..15, one fp16 scale and one integer
zero-point (held as fp16) per output row, two codes per byte along K with the
even k in the low nibble.  Dequantisation is W_hat = (q - z) * s.
"""

import numpy as np

from .numerics import fp16_to_f64


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; byte m holds k = 2m (low) and 2m+1 (high)."""
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    q[..., 0::2] = p & 0x0F
    q[..., 1::2] = p >> 4
    return q


def pack_codes(q: np.ndarray) -> np.ndarray:
    """[..., K] codes in 0..15 -> [..., K/2] bytes (inverse of unpack_codes)."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    if q.size and q.max() > 15:
        raise ValueError("codes must lie in 0..15")
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def dequantize(packed: np.ndarray, s_bits: np.ndarray, z_bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """W_hat[n, k] = (q[n, k] - z[n]) * s[n].

    With integer z the product has at most 15 significant bits, so it is exact
    in fp32 as well as fp64; a non-integer z is handled by the same formula.
    """
    q = unpack_codes(packed).astype(dtype)
    s = fp16_to_f64(s_bits).astype(dtype)[..., None]
    z = fp16_to_f64(z_bits).astype(dtype)[..., None]
    q -= z
    q *= s
    return q


def quantize(W: np.ndarray):
    """Encode fp32 rows: returns (packed codes, scale fp16 bits, zero fp16 bits).

    Per row: the range [lo, hi] is widened to include 0; s = fp16((hi-lo)/15),
    replaced by 1 when it rounds to 0; z = clip(rint(-lo/s), 0, 15);
    q = clip(rint(W/s) + z, 0, 15).  Arithmetic in fp32, rint ties to even.
    """
    W = np.asarray(W, dtype=np.float32)
    n_rows = W.shape[0]
    s_out = np.empty(n_rows, dtype=np.float16)
    z_out = np.empty(n_rows, dtype=np.float16)
    q_out = np.empty(W.shape, dtype=np.uint8)
    for n in range(n_rows):
        row = W[n]
        lo = min(np.float32(row.min()), np.float32(0.0))
        hi = max(np.float32(row.max()), np.float32(0.0))
        s16 = np.float16(np.float32(hi - lo) / np.float32(15.0))
        if s16 == 0:
            s16 = np.float16(1.0)
        s32 = np.float32(s16)
        z = np.float32(min(max(np.rint(np.float32(-lo) / s32), 0.0), 15.0))
        s_out[n], z_out[n] = s16, np.float16(z)
        q_out[n] = encode_with(row[None, :], np.array([s16]).view(np.uint16), np.array([np.float16(z)]).view(np.uint16))[0]
    return pack_codes(q_out), s_out.view(np.uint16), z_out.view(np.uint16)


def encode_with(W: np.ndarray, s_bits: np.ndarray, z_bits: np.ndarray) -> np.ndarray:
    """Codes of W for a given per-row (s, z): clip(rint(W/s) + z, 0, 15), fp32."""
    W = np.asarray(W, dtype=np.float32)
    s = np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.float16).astype(np.float32)[:, None]
    z = np.ascontiguousarray(z_bits, dtype=np.uint16).view(np.float16).astype(np.float32)[:, None]
    q = np.rint(W / s) + z
    return np.clip(q, 0, 15).astype(np.uint8)
