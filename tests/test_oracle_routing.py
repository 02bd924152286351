"""Pins of the oracle's routing (CPU only).

Each test checks the oracle against something other than itself: numbers
printed on the pages, hand-worked cases, exhaustive search on tiny inputs,
and invariants that the routing rule fixes.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from expert_routing_grouped_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_page_printed_no_eplb_numbers():
    """The four numbers printed for placement by expert number, without EPLB."""
    g = _load("page_eplb_no_eplb.json")
    p = g["inputs"]
    scores = W.page_simulation_scores(T=p["T"], E=p["E"], seed=p["seed"])
    ids, _ = oracle.route_grouped(scores, p["top_k"], p["num_groups"], p["topk_groups"])
    load = np.bincount(ids.ravel(), minlength=p["E"]).astype(float)
    for case in g["cases"]:
        per = p["E"] // case["gpus"]
        gpu_load = load.reshape(case["gpus"], per).sum(axis=1)
        assert f"{gpu_load.max() / gpu_load.mean():.2f}" == case["busiest_over_mean"]
        node_of_expert = (np.arange(p["E"]) // per) // (case["gpus"] // case["nodes"])
        touched = [len(set(node_of_expert[row].tolist())) for row in ids[: p["tokens_for_nodes"]]]
        assert f"{np.mean(touched):.2f}" == case["nodes_per_token"]


@pytest.mark.parametrize("case", _load("router_handcrafted.json")["cases"], ids=lambda c: c["name"])
def test_handcrafted_cases(case):
    g = _load("router_handcrafted.json")
    s = np.array([case["scores"]], dtype=np.float32)
    ids, w = oracle.route_grouped(s, case["top_k"], g["num_groups"], case["topk_groups"],
                                  case["renormalize"])
    assert ids[0].tolist() == case["ids"], case["why"]
    np.testing.assert_allclose(w[0], case["weights"], rtol=1e-6, atol=0)


def _brute_force(s, top_k, num_groups, topk_groups):
    """Exhaustive search: the kept groups maximise the sum of group scores, where a group's
    score is its best pair sum; the experts maximise the score sum inside the kept groups.
    Valid for distinct values."""
    E = len(s)
    G = E // num_groups
    gscore = [max(s[g * G + a] + s[g * G + b] for a, b in itertools.combinations(range(G), 2))
              for g in range(num_groups)]
    best_groups = max(itertools.combinations(range(num_groups), topk_groups),
                      key=lambda c: sum(gscore[g] for g in c))
    cand = [e for g in best_groups for e in range(g * G, (g + 1) * G)]
    best = max(itertools.combinations(cand, top_k), key=lambda c: sum(s[e] for e in c))
    return set(best_groups), set(best)


@pytest.mark.parametrize("E,num_groups,topk_groups,top_k", [
    (8, 4, 2, 3), (12, 4, 2, 4), (12, 3, 1, 2), (16, 4, 3, 5), (16, 8, 4, 4), (10, 5, 2, 4)])
def test_brute_force_tiny(E, num_groups, topk_groups, top_k):
    rng = np.random.default_rng(E * 100 + top_k)
    for _ in range(40):
        s = rng.random(E).astype(np.float32)          # distinct values and pair sums (almost surely)
        ids, w = oracle.route_grouped(s[None], top_k, num_groups, topk_groups, True)
        groups, experts = _brute_force(s.astype(float).tolist(), top_k, num_groups, topk_groups)
        assert set(ids[0].tolist()) == experts
        G = E // num_groups
        assert {e // G for e in ids[0].tolist()} <= groups
        # slots are in descending score order
        assert np.all(np.diff(s[ids[0]]) < 0)


def test_single_group_is_plain_topk():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((50, 32)).astype(np.float32)
    s[:, 7] = s[:, 3]          # some equal values
    ids, _ = oracle.route_grouped(s, 6, 1, 1, False)
    for t in range(50):
        expect = sorted(range(32), key=lambda e: (-float(s[t, e]), e))[:6]
        assert ids[t].tolist() == expect


@pytest.mark.parametrize("name", ["route_permute", "prefill_literal"])
def test_invariants_on_workloads(name):
    wl = W.WORKLOADS[name]
    inp = W.generate(wl, with_ffn=False)
    ids, w = oracle.route_grouped(inp.scores, wl.top_k, wl.num_groups, wl.topk_groups, True)
    T, k = ids.shape
    G = wl.E // wl.num_groups
    assert (T, k) == (wl.T, wl.top_k)
    for row in ids:
        assert len(set(row.tolist())) == k                              # k distinct experts
        assert len({e // G for e in row.tolist()}) <= wl.topk_groups     # at most topk_groups groups
    assert np.bincount(ids.ravel(), minlength=wl.E).sum() == T * k        # sum of counts = T k
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)
    assert np.all(np.diff(np.take_along_axis(inp.scores, ids, axis=1), axis=1) <= 0)


def test_prefill_straggler_group_is_group_1():
    """The prefill share owns the expert group with the most assignments (experts 32-63 at seed 0)."""
    wl = W.WORKLOADS["prefill_straggler"]
    inp = W.generate(wl, with_ffn=False)
    ids, _ = oracle.route_grouped(inp.scores, wl.top_k, wl.num_groups, wl.topk_groups, True)
    per_group = np.bincount(ids.ravel() // (wl.E // wl.num_groups), minlength=wl.num_groups)
    g = int(np.argmax(per_group))
    assert g * (wl.E // wl.num_groups) == wl.expert_begin == 32


def test_decode_routing_is_prefix_of_route_permute():
    a = W.generate(W.WORKLOADS["route_permute"], with_ffn=False).scores
    b = W.generate(W.WORKLOADS["decode_ep"], with_ffn=False).scores
    c = W.generate(W.WORKLOADS["decode_tp"], with_ffn=False).scores
    assert np.array_equal(a[:512], b) and np.array_equal(b, c)


def test_softmax_closed_form():
    """logits ln(1..4): probabilities are 1/10 .. 4/10; top-2 picks experts 3, 2."""
    logits = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    ids, w = oracle.route_softmax_topk(logits, 2)
    assert ids[0].tolist() == [3, 2]
    np.testing.assert_allclose(w[0], [0.4, 0.3], rtol=1e-6)
    ids, w = oracle.route_softmax_topk(logits, 2, renormalize=True)
    np.testing.assert_allclose(w[0], [4 / 7, 3 / 7], rtol=1e-6)
    # all experts selected: the probabilities sum to one
    rng = np.random.default_rng(0)
    lg = rng.standard_normal((20, 8)).astype(np.float32)
    _, w = oracle.route_softmax_topk(lg, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)
    # equal logits: uniform probabilities, lowest indices first
    ids, w = oracle.route_softmax_topk(np.zeros((1, 8), np.float32), 3)
    assert ids[0].tolist() == [0, 1, 2]
    np.testing.assert_allclose(w[0], [1 / 8] * 3, rtol=1e-12)


def test_tie_stress_properties():
    s = W.tie_stress_scores(300, 64)
    ids, _ = oracle.route_grouped(s, 8, 8, 4, False)
    G = 8
    for t in range(300):
        row = s[t]
        gs = [np.float32(np.sort(row[g * G:(g + 1) * G])[-1] + np.sort(row[g * G:(g + 1) * G])[-2])
              for g in range(8)]
        kept = sorted(range(8), key=lambda g: (-float(gs[g]), g))[:4]
        cand = [e for e in range(64) if e // G in kept]
        expect = sorted(cand, key=lambda e: (-float(row[e]), e))[:8]
        assert ids[t].tolist() == expect
    assert math.copysign(1.0, float(s[s == 0][0])) in (1.0, -1.0)


def test_invalid_arguments():
    s = np.zeros((2, 16), np.float32)
    with pytest.raises(ValueError):
        oracle.route_grouped(s, 9, 4, 2, True)       # 9 > 2 groups * 4 experts
    with pytest.raises(ValueError):
        oracle.route_grouped(s, 2, 5, 2, True)       # 16 % 5 != 0
    with pytest.raises(ValueError):
        oracle.route_grouped(s, 2, 4, 5, True)       # more kept groups than groups
