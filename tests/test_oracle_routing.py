"""Pins of the oracle's router, top-k selection and regrouping (CPU only)."""

import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth


def _bits(values):
    return synth.bf16_bits_from_f32(np.asarray(values, dtype=np.float32))


def test_hand_worked_routing():
    # x = [1, 2]; rows of W_r give logits [1, 2, 3, 1.5]; top-2 = experts 2 then 1
    x = _bits([[1.0, 2.0]])
    Wr = np.array([[1, 0], [0, 1], [1, 1], [0.5, 0.5]], np.float32)
    logits, idx, w = oracle.route(x, Wr, None, 2)
    assert logits.tolist() == [[1.0, 2.0, 3.0, 1.5]]
    assert idx.tolist() == [[2, 1]]
    e = math.exp(-1.0)
    assert w[0, 0] == pytest.approx(1 / (1 + e), abs=1e-15)
    assert w[0, 1] == pytest.approx(e / (1 + e), abs=1e-15)
    # bias shifts the choice: +2 on expert 3 makes it the top
    _, idx_b, _ = oracle.route(x, Wr, np.array([0, 0, 0, 2], np.float32), 2)
    assert idx_b.tolist() == [[3, 2]]


def test_ties_go_to_lower_expert_id():
    logits = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0], [-1.0, 5.0, -1.0, -1.0]])
    assert oracle.select_topk(logits, 2).tolist() == [[1, 2], [0, 1], [1, 0]]
    assert oracle.select_topk(logits, 3).tolist() == [[1, 2, 3], [0, 1, 2], [1, 0, 2]]


def test_zero_router_gives_first_k_and_uniform_weights():
    rng = np.random.default_rng(0)
    x = _bits(rng.standard_normal((9, 32)))
    for E, k in ((8, 2), (64, 6), (5, 5)):
        _, idx, w = oracle.route(x, np.zeros((E, 32), np.float32), np.zeros(E, np.float32), k)
        assert np.all(idx == np.arange(k)[None, :])
        assert np.all(w == 1.0 / k)


def test_k_equal_E_gives_the_full_softmax():
    rng = np.random.default_rng(1)
    x = _bits(rng.standard_normal((7, 16)))
    Wr = rng.standard_normal((6, 16)).astype(np.float32)
    logits, idx, w = oracle.route(x, Wr, None, 6)
    full = softmax(logits, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, idx.astype(np.int64), 1), rtol=1e-13, atol=0)
    assert np.all(np.sort(idx, axis=1) == np.arange(6))


def test_logits_are_exact_products_summed():
    # a single nonzero term: the logit is exactly the bf16 x fp32 product
    x = _bits([[3.0, 0.0]])
    Wr = np.array([[np.float32(1 / 3), 0.0]], np.float32)
    assert oracle.router_logits(x, Wr)[0, 0] == 3.0 * float(np.float32(1 / 3))


@pytest.mark.parametrize("name", ["tiny", "fine_tiny", "phi35_skew_small"])
def test_topk_against_pure_python_sort(name):
    if name == "phi35_skew_small":
        rng = np.random.default_rng(5)
        x = _bits(rng.standard_normal((40, 64)))
        Wr = (rng.standard_normal((16, 64)) / 8).astype(np.float32)
        b = (-1.2 * np.log(np.arange(1, 17))).astype(np.float32)
        k = 2
    else:
        case = synth.make_case(name)
        x, Wr, b, k = case.hidden, case.weights.router_w, case.weights.router_b, case.shape.top_k
    logits, idx, w = oracle.route(x, Wr, b, k)
    E = Wr.shape[0]
    for t in range(x.shape[0]):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        assert idx[t].tolist() == order
        sel = [logits[t, e] for e in order]
        den = sum(math.exp(v - sel[0]) for v in sel)
        assert w[t].tolist() == pytest.approx([math.exp(v - sel[0]) / den for v in sel], abs=1e-15)
    assert np.all(np.abs(w.sum(axis=1) - 1) <= 1e-12)
    assert np.all(np.diff(np.take_along_axis(logits, idx.astype(np.int64), 1), axis=1) <= 0)
    for row in idx:
        assert len(set(row.tolist())) == k


def test_hand_worked_regroup():
    idx = np.array([[1, 0], [1, 2]], np.int32)          # assignments a = 0..3 -> experts 1, 0, 1, 2
    counts, offsets, perm, inv = oracle.regroup(idx, 3)
    assert counts.tolist() == [1, 2, 1]
    assert offsets.tolist() == [0, 1, 3, 4]
    assert perm.tolist() == [1, 0, 2, 3]
    assert inv.tolist() == [1, 0, 2, 3]


@pytest.mark.parametrize("T,E,k,seed", [(16, 8, 2, 0), (64, 16, 2, 1), (33, 64, 6, 2), (1, 4, 4, 3), (0, 8, 2, 4)])
def test_regroup_invariants_and_bucket_brute_force(T, E, k, seed):
    rng = np.random.default_rng(seed)
    # k distinct experts per token, skewed towards low ids
    p = 1.0 / np.arange(1, E + 1)
    idx = np.array([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)],
                   dtype=np.int32).reshape(T, k)
    counts, offsets, perm, inv = oracle.regroup(idx, E)
    R = T * k
    assert counts.sum() == R
    assert offsets[0] == 0 and offsets[-1] == R and np.all(np.diff(offsets) == counts)
    assert sorted(perm.tolist()) == list(range(R))           # bijection
    np.testing.assert_array_equal(inv[perm], np.arange(R))   # inv o perm = id
    flat = idx.reshape(-1)
    buckets = [[] for _ in range(E)]
    for a in range(R):                                       # stable bucket sort, by hand
        buckets[flat[a]].append(a)
    assert perm.tolist() == [a for b in buckets for a in b]
    assert counts.tolist() == [len(b) for b in buckets]
