"""Pins of the parity checker (oracle/parity.py and the comparison helpers of
oracle/moe_ref.py) on the CPU: hand-built "GPU" results with planted faults
must fail, and the cases the tolerances allow must pass.

The rules follow the TopK and G(x) definitions of "Mixtral of Experts",
section 2.1: TopK keeps the K largest logits (ties within 1e-4 of the K-th
may go either way), slot 0 holds the largest, and gates are the softmax over
the kept logits.  Hand-worked cases: tests/golden/parity_checker.json.
"""
import json
import os

import numpy as np
import pytest

from oracle import moe_ref, parity

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "parity_checker.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_near_tie_is_the_kth_to_next_gap(golden):
    for case in golden["near_tie"]:
        l = np.array([case["logits"]])
        for k, want in case["by_k"].items():
            got = bool(moe_ref.near_tie_tokens(l, int(k))[0])
            assert got == want, (case["logits"], k)


def test_near_tie_is_strictly_below_eps():
    # a gap of exactly eps (representable: 0.5 vs 0.25 with eps 0.25) is not a tie
    l = np.array([[1.0, 0.5, 0.25]])
    assert not moe_ref.near_tie_tokens(l, 2, eps=0.25)[0]
    assert moe_ref.near_tie_tokens(l, 2, eps=0.2500001)[0]


@pytest.mark.parametrize("i", range(12))
def test_routing_cases(golden, i):
    case = golden["routing"][i]
    l = np.array([case["logits"]])
    rep = parity.check_routing(l, case["K"], np.array([case["idx"]]), np.array([case["gate"]]))
    for key in ("near_ties", "set_mismatch", "order_mismatch", "invalid_choice"):
        assert getattr(rep, key) == case[key], (case["name"], key, rep)
    assert rep.ok == case["ok"], (case["name"], rep)


def test_routing_cases_in_one_batch_add_up(golden):
    cases = golden["routing"]
    l = np.array([c["logits"] for c in cases])
    idx = np.array([c["idx"] for c in cases])
    gate = np.array([c["gate"] for c in cases])
    rep = parity.check_routing(l, 2, idx, gate)
    for key in ("near_ties", "set_mismatch", "order_mismatch", "invalid_choice"):
        assert getattr(rep, key) == sum(c[key] for c in cases), key
    assert not rep.ok


def test_forced_idx_takes_the_gpu_choice_only_on_valid_near_ties(golden):
    by = {c["name"]: c for c in golden["routing"]}
    names = ["near_tie_other_candidate", "near_tie_drops_the_clear_winner", "non_tie_other_set",
             "exact_match"]
    l = np.array([by[n]["logits"] for n in names])
    idx = np.array([by[n]["idx"] for n in names])
    gate = np.array([by[n]["gate"] for n in names])
    rep = parity.check_routing(l, 2, idx, gate)
    assert rep.forced_idx.tolist() == [[0, 2], [0, 1], [0, 1], [0, 1]]


def test_gate_tolerance_edges():
    l = np.array([[4.0, 3.0, 1.0, 0.0]])
    g0 = 1.0 / (1.0 + np.exp(-1.0))
    for off, ok in ((9.9e-6, True), (1.01e-5, False)):
        rep = parity.check_routing(l, 2, np.array([[0, 1]]), np.array([[g0 + off, 1 - g0]]))
        assert rep.ok == ok, off


def test_random_batch_and_planted_faults():
    rng = np.random.default_rng(11)
    T, n, K = 2000, 8, 2
    l = rng.standard_normal((T, n))
    idx = moe_ref.topk_indices(l, K)
    gate = moe_ref.topk_softmax(l, idx)
    rep = parity.check_routing(l, K, idx, gate)
    assert rep.ok and rep.set_mismatch == rep.order_mismatch == rep.invalid_choice == 0
    tie = moe_ref.near_tie_tokens(l, K)
    # plant: the 3rd-ranked expert instead of the 2nd on one clear token
    t = int(np.nonzero(~tie)[0][5])
    bad = idx.copy()
    bad[t, 1] = np.argsort(-l[t], kind="stable")[2]
    rep = parity.check_routing(l, K, bad, gate)
    assert rep.set_mismatch == 1 and not rep.ok
    # plant: swapped slots on a token whose top two are far apart
    gaps = -np.diff(-np.sort(-l, axis=1), axis=1)
    t2 = int(np.nonzero(gaps[:, 0] > 0.1)[0][3])
    sw = idx.copy()
    sw[t2] = sw[t2, ::-1]
    rep = parity.check_routing(l, K, sw, gate[:, ::-1] * 0 + np.take_along_axis(
        moe_ref.dense_gate(l, K), sw, axis=1))
    assert rep.order_mismatch == 1 and rep.set_mismatch == 0 and not rep.ok


def test_compare_outputs_hand_value(golden):
    for case in golden["compare_outputs"]:
        mx, mean, rms = moe_ref.compare_outputs(np.array(case["y_ref"]), np.array(case["y_test"]))
        assert mx == pytest.approx(case["max_rel"], rel=1e-15)
        assert mean == pytest.approx(case["mean_rel"], rel=1e-15)
        assert rms == pytest.approx(case["rms"], rel=1e-15)


def test_output_thresholds():
    y = np.ones((10, 100))  # RMS 1
    for d, ok in ((0.019, True), (0.021, False)):  # one entry off: max/RMS = d, mean tiny
        t = y.copy()
        t[3, 7] += d
        rep = parity.check_output(y, t)
        assert rep.max_rel == pytest.approx(d) and rep.ok == ok
    for d, ok in ((0.0019, True), (0.0021, False)):  # every entry off: mean/RMS = max/RMS = d
        rep = parity.check_output(y, y + d)
        assert rep.mean_rel == pytest.approx(d) and rep.ok == ok
    # the RMS is the oracle's: scaling the test output does not loosen the bound
    rep = parity.check_output(y, 1.5 * y)
    assert rep.mean_rel == pytest.approx(0.5) and not rep.ok


def test_output_rejects_non_finite_and_shape_mismatch():
    y = np.ones((4, 8))
    t = y.copy()
    t[1, 1] = np.nan
    assert not parity.check_output(y, t).ok
    t[1, 1] = np.inf
    assert not parity.check_output(y, t).ok
    with pytest.raises(ValueError):
        parity.check_output(y, y[:, :4])
