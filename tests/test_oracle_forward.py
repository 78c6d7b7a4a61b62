"""Pins of the oracle's layer forward (CPU only)."""

import dataclasses
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import assert_out_close, weights_kwargs


def silu(z):
    return z / (1.0 + math.exp(-z))


def _hand_layer():
    """Two experts, d = d_ff = 2.  Expert 0: s = 1, z = 8; expert 1: s = 0.5, z = 4."""
    one, half = np.uint16(0x3C00), np.uint16(0x3800)
    z8 = np.float16(8).view(np.uint16)
    z4 = np.float16(4).view(np.uint16)
    P = oracle.pack_codes
    w = dict(
        w_gate=np.stack([P(np.array([[10, 8], [7, 8]], np.uint8)),      # [[2, 0], [-1, 0]]
                         P(np.array([[4, 6], [4, 5]], np.uint8))]),     # [[0, 1], [0, 0.5]]
        w_up=np.stack([P(np.array([[9, 8], [11, 8]], np.uint8)),        # [[1, 0], [3, 0]]
                       P(np.array([[4, 8], [4, 2]], np.uint8))]),       # [[0, 2], [0, -1]]
        w_down=np.stack([P(np.array([[9, 9], [8, 10]], np.uint8)),      # [[1, 1], [0, 2]]
                         P(np.array([[2, 4], [5, 7]], np.uint8))]),     # [[-1, 0], [0.5, 1.5]]
    )
    for m in ("gate", "up", "down"):
        w["s_" + m] = np.array([[one, one], [half, half]], np.uint16)
        w["z_" + m] = np.array([[z8, z8], [z4, z4]], np.uint16)
    hidden = synth.bf16_bits_from_f32(np.array([[1, 0], [0, 1]], np.float32))
    return hidden, w


def test_hand_worked_forward_top1_and_top2():
    hidden, w = _hand_layer()
    Wr = np.eye(2, dtype=np.float32)
    slots = np.array([0, 1], np.int32)
    # token 0 -> expert 0: G = [2, -1], U = [1, 3], H = [silu(2), 3 silu(-1)], Y = [H0 + H1, 2 H1]
    h0, h1 = silu(2.0), 3 * silu(-1.0)
    ffn0_x0 = [h0 + h1, 2 * h1]
    # token 1 -> expert 1: G = [1, 0.5], U = [2, -1], H = [2 silu(1), -silu(0.5)], Y = [-H0, 0.5 H0 + 1.5 H1]
    g0, g1 = 2 * silu(1.0), -silu(0.5)
    ffn1_x1 = [-g0, 0.5 * g0 + 1.5 * g1]
    r1 = oracle.forward(hidden, Wr, None, slots, top_k=1, **w)
    np.testing.assert_allclose(r1["out"], [ffn0_x0, ffn1_x1], rtol=1e-15, atol=1e-15)
    assert r1["topk_idx"].tolist() == [[0], [1]] and r1["topk_w"].tolist() == [[1.0], [1.0]]
    # top-2: each token's second expert sees G = 0, so it adds exactly zero
    r2 = oracle.forward(hidden, Wr, None, slots, top_k=2, **w)
    a = math.e / (math.e + 1)
    np.testing.assert_allclose(r2["out"], [[a * v for v in ffn0_x0], [a * v for v in ffn1_x1]],
                               rtol=1e-14, atol=1e-15)
    # the same layer with the two experts' slots swapped
    w_sw = {key: v[::-1].copy() for key, v in w.items()}
    r3 = oracle.forward(hidden, Wr, None, np.array([1, 0], np.int32), top_k=1, **w_sw)
    np.testing.assert_array_equal(r3["out"], r1["out"])


@pytest.mark.parametrize("name", ["tiny", "fine_tiny"])
def test_regrouped_forward_equals_dense_then_mask(name):
    case = synth.make_case(name)
    kw = weights_kwargs(case.weights)
    res = oracle.forward(case.hidden, top_k=case.shape.top_k, **kw)
    dense = oracle.brute_dense(case.hidden, top_k=case.shape.top_k, **kw)
    assert_out_close(res["out"], dense, rel=1e-12)
    assert np.all(np.isfinite(res["out"]))            # poisoned slots never reached


def test_single_expert_is_a_dense_swiglu_ffn():
    """E = 1, k = 1: the layer is one dense SwiGLU FFN (torch's CPU silu)."""
    torch = pytest.importorskip("torch")
    shape = synth.LayerShape(12, 128, 256, 1, 1, 1, "identity", 0.0)
    w = synth.make_weights(shape, seed=7)
    x = synth.make_hidden(12, 128, seed=7)
    res = oracle.forward(x, top_k=1, **weights_kwargs(w))
    assert np.all(res["topk_w"] == 1.0)

    def deq(p, s, z):
        p = torch.from_numpy(p[0].astype(np.int64))
        q = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], -1).double()
        s = torch.from_numpy(s[0].view(np.float16).astype(np.float64))[:, None]
        z = torch.from_numpy(z[0].view(np.float16).astype(np.float64))[:, None]
        return (q - z) * s

    xt = torch.from_numpy((x.astype(np.int32) << 16).view(np.float32).astype(np.float64))
    Wg, Wu, Wd = deq(w.w_gate, w.s_gate, w.z_gate), deq(w.w_up, w.s_up, w.z_up), deq(w.w_down, w.s_down, w.z_down)
    ref = (torch.nn.functional.silu(xt @ Wg.T) * (xt @ Wu.T)) @ Wd.T
    assert_out_close(res["out"], ref.numpy(), rel=1e-12)


def test_codes_equal_to_zero_points_give_exact_zero():
    case = synth.make_case("tiny")
    w = dataclasses.replace(case.weights)
    for m in ("gate", "up", "down"):
        z = getattr(w, "z_" + m).view(np.float16).astype(np.uint8)      # integer zero-points
        K2 = getattr(w, "w_" + m).shape[-1]
        q = np.repeat(z[:, :, None], 2 * K2, axis=2)
        setattr(w, "w_" + m, oracle.pack_codes(q))
    res = oracle.forward(case.hidden, top_k=2, **weights_kwargs(w))
    assert np.all(res["out"] == 0)


@pytest.mark.parametrize("which", ["s_down", "s_up"])
def test_doubling_a_linear_scale_doubles_the_output_exactly(which):
    case = synth.make_case("tiny")
    kw = weights_kwargs(case.weights)
    base = oracle.forward(case.hidden, top_k=2, **kw)["out"]
    kw2 = dict(kw)
    kw2[which] = (kw[which].astype(np.uint32) + 0x0400).astype(np.uint16)   # fp16 exponent + 1
    assert np.all(kw2[which].view(np.float16) == 2 * kw[which].view(np.float16))
    np.testing.assert_array_equal(oracle.forward(case.hidden, top_k=2, **kw2)["out"], 2 * base)


def test_gate_and_up_are_not_interchangeable():
    """Swapping W_gate and W_up changes the output (silu acts on the gate only)."""
    case = synth.make_case("tiny")
    kw = weights_kwargs(case.weights)
    base = oracle.forward(case.hidden, top_k=2, **kw)["out"]
    sw = dict(kw, w_gate=kw["w_up"], w_up=kw["w_gate"], s_gate=kw["s_up"], s_up=kw["s_gate"],
              z_gate=kw["z_up"], z_up=kw["z_gate"])
    assert np.abs(oracle.forward(case.hidden, top_k=2, **sw)["out"] - base).max() > 1e-3


def test_slot_permutation_invariance():
    case = synth.make_case("fine_tiny")
    kw = weights_kwargs(case.weights)
    base = oracle.forward(case.hidden, top_k=6, **kw)["out"]
    S = kw["w_gate"].shape[0]
    pi = np.random.default_rng(11).permutation(S)
    kw2 = dict(kw)
    for a in ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up", "z_up", "s_down", "z_down"):
        moved = np.empty_like(kw[a])
        moved[pi] = kw[a]
        kw2[a] = moved
    kw2["slot_table"] = pi[kw["slot_table"]].astype(np.int32)
    np.testing.assert_array_equal(oracle.forward(case.hidden, top_k=6, **kw2)["out"], base)


def test_out_of_range_slot_contributes_zero():
    case = synth.make_case("tiny")
    kw = weights_kwargs(case.weights)
    kw["slot_table"] = kw["slot_table"].copy()
    kw["slot_table"][3] = kw["w_gate"].shape[0]          # one past the pool
    res = oracle.forward(case.hidden, top_k=2, **kw)
    dense = oracle.brute_dense(case.hidden, top_k=2, **kw)
    assert_out_close(res["out"], dense, rel=1e-12)
    hit = np.any(res["topk_idx"] == 3, axis=1)
    assert hit.any()
    full = oracle.forward(case.hidden, top_k=2, **weights_kwargs(case.weights))["out"]
    assert np.all(res["out"][~hit] == full[~hit])


@pytest.mark.parametrize("name", ["tiny", "fine_tiny"])
def test_fp32_and_fp64_paths_agree(name):
    case = synth.make_case(name)
    kw = weights_kwargs(case.weights)
    r64 = oracle.forward(case.hidden, top_k=case.shape.top_k, **kw)
    r32 = oracle.forward(case.hidden, top_k=case.shape.top_k, precision="f32", **kw)
    assert_out_close(r32["out"], r64["out"], rel=1e-5)
    np.testing.assert_array_equal(r32["topk_idx"], r64["topk_idx"])


def test_token_subset_matches_full_forward():
    case = synth.make_case("fine_tiny")
    kw = weights_kwargs(case.weights)
    full = oracle.forward(case.hidden, top_k=6, **kw)["out"]
    sub = oracle.forward(case.hidden, top_k=6, tokens=np.array([0, 5, 15]), **kw)["out"]
    assert_out_close(sub, full[[0, 5, 15]], rel=1e-12)     # BLAS blocking depends on the row count


# ---- shared experts (Strata page, section 2.1: a shared expert kept resident) ----

def test_hand_worked_shared_expert_with_top1():
    """One routed expert (the hand layer's expert 0, top-1, so weight 1) plus
    the hand layer's expert 1 as a shared expert.  Token 0: FFN_0(x0) + FFN_1(x0),
    and FFN_1(x0) = 0 (its gate rows see G = 0); token 1: FFN_0(x1) = 0 plus
    FFN_1(x1)."""
    hidden, w = _hand_layer()
    Wr = np.array([[1.0, 0.0]], np.float32)
    h0, h1 = silu(2.0), 3 * silu(-1.0)
    g0, g1 = 2 * silu(1.0), -silu(0.5)
    want = [[h0 + h1, 2 * h1], [-g0, 0.5 * g0 + 1.5 * g1]]
    r = oracle.forward(hidden, Wr, None, np.array([0, 1], np.int32), top_k=1, num_shared=1, **w)
    np.testing.assert_allclose(r["out"], want, rtol=1e-15, atol=1e-15)
    assert r["topk_idx"].tolist() == [[0, 1], [0, 1]]
    assert r["topk_w"].tolist() == [[1.0, 1.0], [1.0, 1.0]]
    assert r["counts"].tolist() == [2, 2] and r["offsets"].tolist() == [0, 2, 4]
    assert r["perm"].tolist() == [0, 2, 1, 3] and r["inv"].tolist() == [0, 2, 1, 3]


@pytest.mark.parametrize("name", ["shared_tiny", "fine_shared_tiny"])
def test_shared_forward_equals_dense_then_mask(name):
    case = synth.make_case(name)
    kw = weights_kwargs(case.weights)
    k, ns = case.shape.top_k, case.shape.num_shared
    res = oracle.forward(case.hidden, top_k=k, num_shared=ns, **kw)
    dense = oracle.brute_dense(case.hidden, top_k=k, num_shared=ns, **kw)
    assert_out_close(res["out"], dense, rel=1e-12)
    E, T = case.shape.num_experts, case.shape.T
    # every token holds the shared experts in its last columns, with weight 1
    assert res["topk_idx"].shape == (T, k + ns)
    assert np.all(res["topk_idx"][:, k:] == np.arange(E, E + ns))
    assert np.all(res["topk_w"][:, k:] == 1.0)
    assert np.all(res["topk_idx"][:, :k] < E)
    # each shared group holds all T tokens in token order
    for s in range(ns):
        g = res["perm"][res["offsets"][E + s]:res["offsets"][E + s + 1]]
        assert g.tolist() == [t * (k + ns) + k + s for t in range(T)]
    assert res["counts"].sum() == T * (k + ns)


def test_shared_expert_with_zero_weights_adds_nothing():
    case = synth.make_case("shared_tiny")
    kw = weights_kwargs(case.weights)
    sl = int(kw["slot_table"][case.shape.num_experts])
    kw = {a: (v.copy() if isinstance(v, np.ndarray) else v) for a, v in kw.items()}
    for m in ("gate", "up", "down"):
        z = kw["z_" + m][sl].view(np.float16).astype(np.uint8)
        kw["w_" + m][sl] = oracle.pack_codes(np.repeat(z[:, None], 2 * kw["w_" + m].shape[-1], axis=1))
    with_shared = oracle.forward(case.hidden, top_k=1, num_shared=1, **kw)["out"]
    routed_only = oracle.forward(case.hidden, top_k=1, **dict(kw, slot_table=kw["slot_table"][:-1]))["out"]
    np.testing.assert_array_equal(with_shared, routed_only)


def test_shared_copy_of_the_only_expert_doubles_the_output():
    """E = 1, top-1 (weight 1) and a shared expert in the same slot: exactly twice
    the routed-only output."""
    shape = synth.LayerShape(12, 128, 256, 1, 1, 1, "identity", 0.0)
    w = synth.make_weights(shape, seed=3)
    x = synth.make_hidden(12, 128, seed=3)
    kw = weights_kwargs(w)
    base = oracle.forward(x, top_k=1, **kw)["out"]
    both = oracle.forward(x, top_k=1, num_shared=1, **dict(kw, slot_table=np.array([0, 0], np.int32)))["out"]
    np.testing.assert_array_equal(both, 2 * base)


def test_shared_count_must_match_the_slot_table():
    case = synth.make_case("shared_tiny")
    kw = weights_kwargs(case.weights)
    with pytest.raises(ValueError):
        oracle.forward(case.hidden, top_k=1, **kw)           # slot table has E + 1 entries


# ---- other weight formats (8-bit codes, grouped (s, z)) ----

@pytest.mark.parametrize("name", ["tiny_q4g128", "tiny_q8", "tiny_q8g128"])
def test_format_forward_equals_dense_then_mask(name):
    case = synth.make_case(name)
    sh = case.shape
    kw = weights_kwargs(case.weights)
    fmt = dict(top_k=sh.top_k, num_shared=sh.num_shared, bits=sh.bits, group=sh.group)
    res = oracle.forward(case.hidden, **fmt, **kw)
    dense = oracle.brute_dense(case.hidden, **fmt, **kw)
    assert_out_close(res["out"], dense, rel=1e-12)
    r32 = oracle.forward(case.hidden, precision="f32", **fmt, **kw)
    assert_out_close(r32["out"], res["out"], rel=1e-5)


def test_int8_layer_with_16x_codes_equals_the_int4_layer():
    """q8 = 16 q4, z8 = 16 z4, s8 = s4 / 16 (exact in fp16 at these scales):
    the same weights, so the same output bit for bit."""
    case = synth.make_case("tiny")
    kw = weights_kwargs(case.weights)
    base = oracle.forward(case.hidden, top_k=2, **kw)["out"]
    kw8 = dict(kw)
    for m in ("gate", "up", "down"):
        kw8["w_" + m] = 16 * oracle.unpack_codes(kw["w_" + m])
        s = kw["s_" + m].view(np.float16)
        assert np.all((s / np.float16(16)) * np.float16(16) == s)
        kw8["s_" + m] = (s / np.float16(16)).view(np.uint16)
        kw8["z_" + m] = (kw["z_" + m].view(np.float16) * np.float16(16)).view(np.uint16)
    np.testing.assert_array_equal(oracle.forward(case.hidden, top_k=2, bits=8, **kw8)["out"], base)


def test_grouped_layer_with_row_parameters_equals_the_row_layer():
    case = synth.make_case("tiny")
    kw = weights_kwargs(case.weights)
    base = oracle.forward(case.hidden, top_k=2, **kw)["out"]
    kwg = dict(kw)
    d, f = case.shape.d_model, case.shape.d_ff
    for m, K in (("gate", d), ("up", d), ("down", f)):
        for p in ("s_", "z_"):
            kwg[p + m] = np.repeat(kw[p + m][:, None, :], K // 128, axis=1)   # [S, K/128, N]
    np.testing.assert_array_equal(oracle.forward(case.hidden, top_k=2, group=128, **kwg)["out"], base)
