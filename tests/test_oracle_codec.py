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


# ---- 8-bit codes and grouped (s, z) (Co-inference page, section 5.1) ----

def _f16bits(vals):
    return np.array(vals, np.float16).view(np.uint16)


def test_8bit_dequantize_closed_form():
    # s = 0.5, z = 128: q = 255 -> 63.5, 128 -> 0, 0 -> -64, 129 -> 0.5
    q = np.array([[255, 128, 0, 129]], np.uint8)
    assert oracle.pack_codes(q, 8).tolist() == q.tolist()          # one code per byte
    W = oracle.dequantize(q, _f16bits([0.5]), _f16bits([128]), bits=8)
    assert W.tolist() == [[63.5, 0.0, -64.0, 0.5]]


def test_grouped_dequantize_closed_form_and_layout():
    """K = 4 in groups of 2; parameters are [K/G][N] (group-major)."""
    q = np.array([[9, 7, 4, 2],
                  [8, 8, 15, 0]], np.uint8)
    # row 0: group 0 (s=1, z=8), group 1 (s=0.5, z=0); row 1: group 0 (s=2, z=8), group 1 (s=0.25, z=15)
    s = _f16bits([[1.0, 2.0], [0.5, 0.25]])
    z = _f16bits([[8, 8], [0, 15]])
    W = oracle.dequantize(oracle.pack_codes(q), s, z, group=2)
    assert W.tolist() == [[1.0, -1.0, 2.0, 1.0], [0.0, 0.0, 0.0, -3.75]]


@pytest.mark.parametrize("bits", [4, 8])
def test_groups_sharing_the_row_parameters_equal_the_per_row_format(bits):
    rng = np.random.default_rng(5)
    N, K, G = 6, 512, 128
    q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.01, 1, size=N).astype(np.float16).view(np.uint16)
    z = rng.integers(0, 1 << bits, size=N).astype(np.float16).view(np.uint16)
    row = oracle.dequantize(oracle.pack_codes(q, bits), s, z, bits=bits)
    grp = oracle.dequantize(oracle.pack_codes(q, bits), np.tile(s, (K // G, 1)), np.tile(z, (K // G, 1)),
                            bits=bits, group=G)
    np.testing.assert_array_equal(grp, row)


def test_8bit_codes_16x_the_int4_codes_dequantise_identically():
    """q8 = 16 q4, z8 = 16 z4, s8 = s4 / 16 describe the same weights exactly."""
    rng = np.random.default_rng(6)
    q4 = rng.integers(0, 16, size=(5, 256), dtype=np.uint8)
    s4 = (2.0 ** rng.integers(-8, 0, size=5)).astype(np.float16)
    z4 = rng.integers(0, 16, size=5).astype(np.float16)
    W4 = oracle.dequantize(oracle.pack_codes(q4), s4.view(np.uint16), z4.view(np.uint16))
    W8 = oracle.dequantize(16 * q4, (s4 / 16).view(np.uint16), (z4 * 16).view(np.uint16), bits=8)
    np.testing.assert_array_equal(W8, W4)


@pytest.mark.parametrize("bits,group", [(8, 0), (4, 128), (8, 128)])
def test_quantize_error_bound_and_roundtrip_other_formats(bits, group):
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((12, 384)) / 16).astype(np.float32)
    W[3] = 0.0
    W[4] = np.abs(W[4])
    packed, s_bits, z_bits = oracle.quantize(W, bits, group)
    qmax = (1 << bits) - 1
    q = oracle.unpack_codes(packed, bits)
    assert q.shape == W.shape and q.max() <= qmax
    pshape = (W.shape[0],) if group == 0 else (W.shape[1] // group, W.shape[0])
    assert s_bits.shape == pshape and z_bits.shape == pshape
    z = z_bits.view(np.float16).astype(np.float64)
    assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= qmax
    Wh = oracle.dequantize(packed, s_bits, z_bits, bits=bits, group=group)
    s = s_bits.view(np.float16).astype(np.float64)
    s_el = s[:, None] if group == 0 else np.repeat(s.T, group, axis=1)
    assert np.all(np.abs(W - Wh) <= 0.51 * s_el)
    np.testing.assert_array_equal(
        oracle.encode_with(oracle.dequantize(packed, s_bits, z_bits, np.float32, bits, group), s_bits, z_bits,
                           bits, group), q)


def test_grouping_confines_an_outlier_to_its_group():
    """The reason the page gives for grouped quantisation: one outlier widens
    the range of its own group only, so the other groups keep their precision."""
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((4, 512)) * 0.02).astype(np.float32)
    W[:, 5] = 3.0                                    # an outlier in group 0 of every row
    err = {}
    for group in (0, 128):
        packed, s, z = oracle.quantize(W, 4, group)
        err[group] = np.abs(oracle.dequantize(packed, s, z, group=group) - W)[:, 128:].max()
    assert err[128] * 10 < err[0]


@pytest.mark.parametrize("name", ["tiny_q4g128", "tiny_q8", "tiny_q8g128"])
def test_generator_codes_follow_the_encoding_rule_other_formats(name):
    case = synth.make_case(name)
    w, shp = case.weights, case.shape
    for e in (0, shp.num_experts - 1):
        slot = int(w.slot_table[e])
        for W, packed, s, z in zip(synth.draw_dense_expert(shp, case.seed, e),
                                   (w.w_gate, w.w_up, w.w_down),
                                   (w.s_gate, w.s_up, w.s_down), (w.z_gate, w.z_up, w.z_down)):
            p2, s2, z2 = oracle.quantize(W, shp.bits, shp.group)
            np.testing.assert_array_equal(p2, packed[slot])
            np.testing.assert_array_equal(s2, s[slot])
            np.testing.assert_array_equal(z2, z[slot])
