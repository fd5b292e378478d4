"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against hand-worked values (tests/golden), a
different evaluation of the same definition (dense over all experts, brute
force over expert subsets, the K = n softmax mixture), a library routine in a
special case (identical experts collapse to one FFN evaluated with matmul), an
invariant (gates sum to one, permutation of expert ids), or a closed form of
the pages (Table 5 repetition rates, the uniform 1/8 share of Figure 7).
"""
import json
import math
import os

import numpy as np
import pytest

import moe_synth
from oracle import moe_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand_layer(rng, T, D, H, n, scale=1.0):
    x = rng.standard_normal((T, D))
    wg = rng.standard_normal((D, n)) * scale
    w1 = rng.standard_normal((n, D, H)) / np.sqrt(D)
    w3 = rng.standard_normal((n, D, H)) / np.sqrt(D)
    w2 = rng.standard_normal((n, H, D)) / np.sqrt(H)
    return x, wg, w1, w3, w2


# --- hand-worked values ------------------------------------------------------
def test_swiglu_hand_examples(golden):
    for case in golden["swiglu"]:
        x = np.array([case["x"]])
        E = moe_ref.swiglu_expert(x, np.array(case["w1"]), np.array(case["w3"]), np.array(case["w2"]))
        np.testing.assert_allclose(E[0], case["E"], rtol=1e-14, atol=0)


def test_gate_hand_examples(golden):
    for case in golden["gate"]:
        l = np.array([case["logits"]])
        idx = moe_ref.topk_indices(l, case["K"])
        assert idx[0].tolist() == case["idx"]
        g = moe_ref.topk_softmax(l, idx)
        np.testing.assert_allclose(g[0], case["gate"], rtol=1e-15, atol=1e-16)


def test_gate_k1_exactly_one(golden):
    rng = np.random.default_rng(3)
    l = rng.standard_normal((1000, 8)) * 30
    g = moe_ref.topk_softmax(l, moe_ref.topk_indices(l, 1))
    assert np.all(g == 1.0)


def test_layer_hand_examples(golden):
    for case in golden["layer"]:
        out = moe_ref.moe_layer(np.array(case["x"]), np.array(case["w_gate"]), np.array(case["w1"]),
                                np.array(case["w3"]), np.array(case["w2"]), case["K"])
        assert out["idx"].tolist() == case["idx"]
        np.testing.assert_allclose(out["gate"], case["gate"], rtol=1e-15)
        np.testing.assert_allclose(out["y"], case["y"], rtol=1e-14)


# --- invariants and special cases -------------------------------------------
def test_gate_rows_sum_to_one_with_k_nonzeros():
    rng = np.random.default_rng(0)
    l = rng.standard_normal((5000, 8)) * 4
    for k in (1, 2, 3, 8):
        g = moe_ref.dense_gate(l, k)
        assert np.all(np.abs(g.sum(axis=1) - 1.0) <= 2e-15)  # a few ulps of summation
        assert np.all((g != 0).sum(axis=1) == k)


def test_topk_is_the_k_largest_and_ordered():
    rng = np.random.default_rng(1)
    l = rng.integers(-3, 4, size=(4000, 8)).astype(float)  # many exact ties
    for k in (1, 2, 4):
        idx = moe_ref.topk_indices(l, k)
        kept = np.take_along_axis(l, idx, 1)
        # slot order: non-increasing logits, equal logits in increasing index
        assert np.all(np.diff(kept, axis=1) <= 0)
        eq = np.diff(kept, axis=1) == 0
        assert np.all(np.diff(idx, axis=1)[eq] > 0)
        # every dropped logit is <= the smallest kept one, and strictly smaller
        # when its index is lower (lowest index wins ties)
        for t in range(200):
            dropped = np.setdiff1d(np.arange(8), idx[t])
            m = kept[t, -1]
            assert np.all(l[t, dropped] <= m)
            assert not np.any((l[t, dropped] == m) & (dropped < idx[t, -1]))


def test_k2_gate_is_sigmoid_of_logit_gap():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((2000, 8)) * 3
    idx = moe_ref.topk_indices(l, 2)
    g = moe_ref.topk_softmax(l, idx)
    kept = np.take_along_axis(l, idx, 1)
    sig = 1.0 / (1.0 + np.exp(-(kept[:, 0] - kept[:, 1])))
    np.testing.assert_allclose(g[:, 0], sig, rtol=1e-14)
    assert np.all(g[:, 0] >= 0.5)


def test_softmax_of_topk_is_renormalised_topk_of_softmax():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((500, 8)) * 2
    for k in (1, 2, 5):
        idx = moe_ref.topk_indices(l, k)
        p = np.exp(l) / np.exp(l).sum(axis=1, keepdims=True)
        pk = np.take_along_axis(p, idx, 1)
        np.testing.assert_allclose(moe_ref.topk_softmax(l, idx), pk / pk.sum(1, keepdims=True), rtol=1e-13)


def test_sparse_equals_dense_masked():
    rng = np.random.default_rng(5)
    x, wg, w1, w3, w2 = _rand_layer(rng, 37, 24, 40, 8)
    for k in (1, 2, 3):
        ys = moe_ref.moe_layer(x, wg, w1, w3, w2, k)["y"]
        yd = moe_ref.moe_layer_dense(x, wg, w1, w3, w2, k)
        np.testing.assert_allclose(ys, yd, rtol=1e-12, atol=1e-13)


def test_k_equals_n_is_dense_softmax_mixture():
    rng = np.random.default_rng(6)
    n = 6
    x, wg, w1, w3, w2 = _rand_layer(rng, 20, 16, 24, n)
    y = moe_ref.moe_layer(x, wg, w1, w3, w2, n)["y"]
    l = x @ wg
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = np.zeros_like(y)
    for e in range(n):
        a, b = x @ w1[e], x @ w3[e]
        ref += p[:, e:e + 1] * (((a * (1 / (1 + np.exp(-a)))) * b) @ w2[e])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_k1_is_argmax_expert():
    rng = np.random.default_rng(7)
    x, wg, w1, w3, w2 = _rand_layer(rng, 25, 12, 20, 5)
    out = moe_ref.moe_layer(x, wg, w1, w3, w2, 1)
    am = np.argmax(x @ wg, axis=1)  # numpy returns the first maximum
    assert np.array_equal(out["idx"][:, 0], am)
    assert np.all(out["gate"] == 1.0)
    for t in range(x.shape[0]):
        e = am[t]
        a, b = x[t] @ w1[e], x[t] @ w3[e]
        np.testing.assert_allclose(out["y"][t], (a / (1 + np.exp(-a)) * b) @ w2[e], rtol=1e-12)


def test_bruteforce_tiny():
    rng = np.random.default_rng(8)
    for (T, D, H, n, k) in ((4, 8, 16, 5, 2), (3, 5, 7, 4, 3), (2, 6, 4, 5, 1)):
        x, wg, w1, w3, w2 = _rand_layer(rng, T, D, H, n)
        yb = moe_ref.moe_layer_bruteforce(x, wg, w1, w3, w2, k)
        ys = moe_ref.moe_layer(x, wg, w1, w3, w2, k)["y"]
        np.testing.assert_allclose(ys, yb, rtol=1e-12, atol=1e-13)


def test_bruteforce_tiny_with_ties():
    # integer-valued x and W_g force exact logit ties; brute force breaks them
    # by lexicographic order of the expert subset, the oracle by lowest index
    rng = np.random.default_rng(9)
    x = rng.integers(-1, 2, size=(4, 3)).astype(float)
    wg = rng.integers(-1, 2, size=(3, 5)).astype(float)
    _, _, w1, w3, w2 = _rand_layer(rng, 4, 3, 6, 5)
    for k in (1, 2, 3):
        yb = moe_ref.moe_layer_bruteforce(x, wg, w1, w3, w2, k)
        ys = moe_ref.moe_layer(x, wg, w1, w3, w2, k)["y"]
        np.testing.assert_allclose(ys, yb, rtol=1e-12, atol=1e-13)


def test_identical_experts_collapse_to_one_ffn():
    rng = np.random.default_rng(10)
    T, D, H, n = 30, 16, 32, 8
    x = rng.standard_normal((T, D))
    wg = rng.standard_normal((D, n))
    W1 = rng.standard_normal((D, H))
    W3 = rng.standard_normal((D, H))
    W2 = rng.standard_normal((H, D))
    w1, w3, w2 = (np.repeat(W[None], n, 0) for W in (W1, W3, W2))
    a = np.matmul(x, W1)
    ref = np.matmul(a * 0.5 * (1 + np.tanh(0.5 * a)) * np.matmul(x, W3), W2)  # z*sigmoid(z)
    for k in (1, 2, 8):
        np.testing.assert_allclose(moe_ref.moe_layer(x, wg, w1, w3, w2, k)["y"], ref, rtol=1e-12, atol=1e-12)


def test_zero_input_gives_zero():
    rng = np.random.default_rng(11)
    _, wg, w1, w3, w2 = _rand_layer(rng, 1, 16, 32, 8)
    out = moe_ref.moe_layer(np.zeros((5, 16)), wg, w1, w3, w2, 2)
    assert np.all(out["y"] == 0.0)
    # all logits tie at 0: experts 0 and 1, half each
    assert out["idx"].tolist() == [[0, 1]] * 5
    assert np.all(out["gate"] == 0.5)


def test_expert_permutation_invariance():
    rng = np.random.default_rng(12)
    x, wg, w1, w3, w2 = _rand_layer(rng, 40, 16, 24, 8)
    perm = rng.permutation(8)
    a = moe_ref.moe_layer(x, wg, w1, w3, w2, 2)
    b = moe_ref.moe_layer(x, wg[:, perm], w1[perm], w3[perm], w2[perm], 2)
    # new expert j is old expert perm[j]
    assert np.array_equal(perm[b["idx"]], a["idx"])
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-12, atol=1e-13)


def test_forced_idx_matches_dense_gate_of_forced_set():
    rng = np.random.default_rng(13)
    x, wg, w1, w3, w2 = _rand_layer(rng, 10, 8, 12, 6)
    forced = np.tile(np.array([[4, 2]]), (10, 1))
    out = moe_ref.moe_layer(x, wg, w1, w3, w2, 2, forced_idx=forced)
    l = x @ wg
    g0 = 1 / (1 + np.exp(-(l[:, 4] - l[:, 2])))
    np.testing.assert_allclose(out["gate"][:, 0], g0, rtol=1e-13)
    ref = np.zeros_like(out["y"])
    for t in range(10):
        for s, e in enumerate((4, 2)):
            a, b = x[t] @ w1[e], x[t] @ w3[e]
            gs = g0[t] if s == 0 else 1 - g0[t]
            ref[t] += gs * ((a / (1 + np.exp(-a)) * b) @ w2[e])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-13)


def test_bf16_inputs_are_widened_exactly():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000], np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38, 0.0, -0.0]
    got = moe_ref.from_bf16(bits)
    assert got.dtype == np.float64
    assert got.tolist() == want
    assert math.copysign(1.0, got[-1]) == -1.0


# --- routing closed forms (section 5) ---------------------------------------
def test_repetition_rates_match_random_assignment_closed_forms(golden):
    cf = golden["routing_closed_forms"]
    rng = np.random.default_rng(14)
    l = rng.standard_normal((200000, 8))
    idx = moe_ref.topk_indices(l, 2)
    first, either = moe_ref.consecutive_repeat(idx)
    assert abs(first - cf["first_choice_repeat"]) < 0.004      # ~5 sigma at N=2e5
    assert abs(either - cf["either_choice_repeat"]) < 0.006
    share = moe_ref.expert_share(idx, 8)
    assert np.all(np.abs(share - cf["uniform_share"]) < 0.003)


def test_repetition_rates_for_many_small_experts():
    # The section-5 rates for K of n experts under random assignment: the next
    # token's first choice matches with probability 1/n, and its K-set misses
    # this token's K-set with probability C(n-K, K) / C(n, K) (both K-sets are
    # uniform K-subsets).  n = 8, K = 2 gives the pages' 1/8 and 1 - (6/8)(5/7);
    # here the fine-grained n = 160, K = 8.
    assert math.isclose(1 - math.comb(6, 2) / math.comb(8, 2), 1 - (6 / 8) * (5 / 7))
    n, K, N = 160, 8, 100000
    rng = np.random.default_rng(16)
    idx = moe_ref.topk_indices(rng.standard_normal((N, n)), K)
    first, either = moe_ref.consecutive_repeat(idx)
    want_either = 1 - math.comb(n - K, K) / math.comb(n, K)
    assert abs(first - 1 / n) < 0.0015                            # ~6 sigma at N=1e5
    assert abs(either - want_either) < 0.008
    share = moe_ref.expert_share(idx, n)
    assert np.all(np.abs(share - 1 / n) < 0.002)


def test_repetition_rate_detects_structure():
    # pairs: (0,1)->(0,2) share first and an expert; (0,2)->(2,3) share expert 2
    # only; (2,3)->(4,5) nothing; (4,5)->(5,4) share experts but not the first
    idx = np.array([[0, 1], [0, 2], [2, 3], [4, 5], [5, 4]])
    first, either = moe_ref.consecutive_repeat(idx)
    assert first == 0.25
    assert either == 0.75


def test_route_stats_counts_agree_with_the_rates_and_a_hand_example(golden):
    # the hand example above, as exact counts
    idx = np.array([[0, 1], [0, 2], [2, 3], [4, 5], [5, 4]])
    st = moe_ref.route_stats(idx, 8)
    assert st["first"] == [2, 0, 1, 0, 1, 1, 0, 0]
    assert st["any"] == [2, 1, 2, 1, 2, 2, 0, 0]
    assert (st["repeat_first"], st["repeat_either"]) == (1, 3)
    # random assignment: counts / denominators are the section-5 rates
    cf = golden["routing_closed_forms"]
    rng = np.random.default_rng(15)
    idx = moe_ref.topk_indices(rng.standard_normal((20000, 8)), 2)
    st = moe_ref.route_stats(idx, 8)
    first, either = moe_ref.consecutive_repeat(idx)
    assert st["repeat_first"] == round(first * (len(idx) - 1))
    assert st["repeat_either"] == round(either * (len(idx) - 1))
    assert np.array_equal(np.array(st["any"]) / idx.size, moe_ref.expert_share(idx, 8))
    assert sum(st["first"]) == len(idx) and sum(st["any"]) == idx.size
    assert abs(st["repeat_either"] / (len(idx) - 1) - cf["either_choice_repeat"]) < 0.02


def test_route_stats_ignores_out_of_range_ids():
    # -1 and 8 are dropped slots: never counted, never matched (not even by
    # another dropped slot)
    idx = np.array([[-1, 3], [-1, 3], [8, 2], [8, 5], [1, -1]])
    st = moe_ref.route_stats(idx, 8)
    assert st["first"] == [0, 1, 0, 0, 0, 0, 0, 0]
    assert st["any"] == [0, 1, 1, 2, 0, 1, 0, 0]
    # t=0->1 share 3 (first choices both dropped: no first repeat); 1->2 none;
    # 2->3 none (8 matches nothing); 3->4 none
    assert (st["repeat_first"], st["repeat_either"]) == (0, 1)
