"""Pins of the oracle's number formats and int4 codec (CPU only)."""

import numpy as np
import pytest

import oracle
import synth


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC040, 0x4049, 0x0000, 0x8000, 0x3F81, 0x7F7F], dtype=np.uint16)
    want = [1.0, -3.0, 3.140625, 0.0, -0.0, 1.0 + 2.0 ** -7, (2 - 2.0 ** -7) * 2.0 ** 127]
    assert oracle.bf16_to_f64(bits).tolist() == want


def test_fp16_decode_matches_numpy():
    bits = np.arange(0, 0x7C00, 7, dtype=np.uint16)
    np.testing.assert_array_equal(oracle.fp16_to_f64(bits), bits.view(np.float16).astype(np.float64))


def test_pack_layout_low_nibble_even_k():
    # byte 0x21 holds k=0 -> 1 (low nibble) and k=1 -> 2 (high nibble)
    assert oracle.unpack_codes(np.array([[0x21, 0xF0]], np.uint8)).tolist() == [[1, 2, 0, 15]]
    assert oracle.pack_codes(np.array([[1, 2, 0, 15]], np.uint8)).tolist() == [[0x21, 0xF0]]


def test_pack_unpack_identity():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(5, 64), dtype=np.uint8)
    np.testing.assert_array_equal(oracle.unpack_codes(oracle.pack_codes(q)), q)
    p = rng.integers(0, 256, size=(3, 17), dtype=np.uint8)
    np.testing.assert_array_equal(oracle.pack_codes(oracle.unpack_codes(p)), p)


def test_dequantize_closed_form():
    # s = 0.5 (fp16 0x3800), z = 8: q=15 -> 3.5, q=8 -> 0, q=0 -> -4
    packed = oracle.pack_codes(np.array([[15, 8, 0, 9]], np.uint8))
    s = np.array([0x3800], np.uint16)
    z = np.array([np.float16(8)], np.float16).view(np.uint16)
    assert oracle.dequantize(packed, s, z).tolist() == [[3.5, 0.0, -4.0, 0.5]]
    # fp32 dequantisation is exact (<= 15 significant bits)
    assert oracle.dequantize(packed, s, z, np.float32).tolist() == [[3.5, 0.0, -4.0, 0.5]]


def test_dequantize_codes_equal_zero_point_give_zero():
    rng = np.random.default_rng(2)
    z = rng.integers(0, 16, size=7)
    q = np.repeat(z[:, None], 32, axis=1).astype(np.uint8)
    s = rng.uniform(0.01, 2, size=7).astype(np.float16).view(np.uint16)
    W = oracle.dequantize(oracle.pack_codes(q), s, z.astype(np.float16).view(np.uint16))
    assert np.all(W == 0)


def test_quantize_error_bound_and_ranges():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((40, 256)) / 16).astype(np.float32)
    W[3] = 0.0                      # all-zero row: s falls back to 1
    W[4] = np.abs(W[4])             # one-signed rows: the range is widened to 0
    W[5] = -np.abs(W[5])
    packed, s_bits, z_bits = oracle.quantize(W)
    q = oracle.unpack_codes(packed)
    s = s_bits.view(np.float16).astype(np.float64)
    z = z_bits.view(np.float16).astype(np.float64)
    assert q.max() <= 15
    assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= 15
    assert s[3] == 1.0 and np.all(q[3] == z[3])
    assert z[4] == 0 and z[5] == 15
    Wh = oracle.dequantize(packed, s_bits, z_bits)
    assert np.all(np.abs(W - Wh) <= 0.51 * s[:, None])


def test_quantize_roundtrip_with_stored_params():
    """Re-encoding W_hat with the stored (s, z) returns the codes exactly."""
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    packed, s_bits, z_bits = oracle.quantize(W)
    Wh = oracle.dequantize(packed, s_bits, z_bits, np.float32)
    np.testing.assert_array_equal(oracle.encode_with(Wh, s_bits, z_bits), oracle.unpack_codes(packed))


@pytest.mark.parametrize("name", ["tiny", "fine_tiny"])
def test_generator_codes_follow_the_encoding_rule(name):
    """The generator's int4 pool equals the oracle's encoder applied to the
    generator's fp32 draws (two independent implementations of one rule)."""
    case = synth.make_case(name)
    w = case.weights
    for e in (0, case.shape.num_experts - 1):
        slot = int(w.slot_table[e])
        for W, packed, s, z in zip(synth.draw_dense_expert(case.shape, case.seed, e),
                                   (w.w_gate, w.w_up, w.w_down),
                                   (w.s_gate, w.s_up, w.s_down), (w.z_gate, w.z_up, w.z_down)):
            p2, s2, z2 = oracle.quantize(W)
            np.testing.assert_array_equal(p2, packed[slot])
            np.testing.assert_array_equal(s2, s[slot])
            np.testing.assert_array_equal(z2, z[slot])
