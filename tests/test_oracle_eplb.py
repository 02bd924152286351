"""Pins of the EPLB placement oracle (page "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠",
section "EPLB 与路由约束"): the eight numbers the page prints for global and hierarchical EPLB,
hand-worked packings and replications, and structural invariants. CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
from expert_routing_grouped_amd import workloads as W
from oracle import eplb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def page_sim():
    g = _golden("page_eplb_placements.json")
    p = g["inputs"]
    scores = W.page_simulation_scores(T=p["T"], E=p["E"], seed=p["seed"])
    ids, _ = oracle.route_grouped(scores, p["top_k"], p["num_groups"], p["topk_groups"])
    load = np.bincount(ids.ravel(), minlength=p["E"]).astype(float)
    return g, ids, load


def test_page_printed_eplb_numbers(page_sim):
    g, ids, load = page_sim
    p = g["inputs"]
    for c in g["cases"]:
        gpus = eplb.place(load, p["num_groups"], c["nodes"], c["gpus"], c["physical"],
                          c["strategy"] == "hierarchical")
        gl = eplb.gpu_loads(load, gpus)
        assert f"{gl.max() / gl.mean():.2f}" == c["busiest_over_mean"], c
        phys = eplb.remap(ids[: p["tokens_for_nodes"]], gpus, c["nodes"])
        npt = eplb.nodes_per_token(phys, len(gpus[0]), c["gpus"] // c["nodes"])
        assert f"{npt.mean():.2f}" == c["nodes_per_token"], c


def test_remap_without_replicas_gives_the_no_eplb_numbers(page_sim):
    # placement by expert number, one replica each: the remap has a single choice
    # per slot, and the node count is the page's no-EPLB figure
    _, ids, _ = page_sim
    g = _golden("page_eplb_no_eplb.json")
    for c in g["cases"]:
        per = 256 // c["gpus"]
        gpus = [list(range(i * per, (i + 1) * per)) for i in range(c["gpus"])]
        phys = eplb.remap(ids[:2000], gpus, c["nodes"])
        assert np.array_equal(phys, ids[:2000])
        npt = eplb.nodes_per_token(phys, per, c["gpus"] // c["nodes"])
        assert f"{npt.mean():.2f}" == c["nodes_per_token"]


def test_balanced_pack_by_hand():
    # weights 5 4 3 3 1 1 into 2 packs of 3: item 0 -> A (5), 1 -> B (4), 2 -> B (7),
    # 3 -> A (8), 4 -> B (8, now full), 5 -> A
    packs = eplb.balanced_pack([5, 4, 3, 3, 1, 1], 2)
    assert packs == [[0, 3, 5], [1, 2, 4]]
    # a full pack takes nothing more even when it is the lightest
    assert eplb.balanced_pack([10, 1, 1, 1], 2) == [[0, 3], [1, 2]]


def test_replicate_by_hand():
    load = np.array([8.0, 3.0, 6.0])
    # per-replica loads (8, 3, 6): add to 0 -> (4, 3, 6): add to 2 -> (4, 3, 3): add to 0
    phys, cnt = eplb.replicate(load, [0, 1, 2], 6)
    assert cnt == {0: 3, 1: 1, 2: 2}
    assert phys == [0, 0, 0, 1, 2, 2]
    # equal loads per replica go to the expert listed first
    phys, cnt = eplb.replicate(np.array([2.0, 4.0, 4.0]), [2, 1, 0], 4)
    assert cnt == {2: 2, 1: 1, 0: 1} and phys == [2, 2, 1, 0]


@pytest.mark.parametrize("hier", [False, True])
def test_place_invariants(page_sim, hier):
    _, _, load = page_sim
    gpus = eplb.place(load, 8, 4, 32, 288, hier)
    assert len(gpus) == 32 and all(len(g) == 9 for g in gpus)
    flat = [e for g in gpus for e in g]
    assert sorted(set(flat)) == list(range(256))
    if hier:   # a group's experts (and their replicas) stay on one node
        node_of = {}
        for gi, g in enumerate(gpus):
            for e in g:
                node_of.setdefault(e // 32, set()).add(gi // 8)
        assert all(len(v) == 1 for v in node_of.values())


def test_remap_picks_replicas_of_the_right_expert(page_sim):
    _, ids, load = page_sim
    gpus = eplb.place(load, 8, 8, 64, 320, False)
    flat = np.array([e for g in gpus for e in g])
    phys = eplb.remap(ids[:500], gpus, 8)
    assert np.array_equal(flat[phys], ids[:500])


def test_remap_by_hand():
    # 2 nodes x 1 GPU x 2 slots: GPU 0 = [A, B], GPU 1 = [A, C] with A = 0, B = 1, C = 2.
    # Token [A, C]: A has no replica on a node in use yet -> the lowest node (slot 0);
    # C only lives on node 1 (slot 3). Token [C, A]: C -> slot 3 puts node 1 in use,
    # so A takes its replica there (slot 2). Token [B, A]: B -> slot 1 (node 0), then
    # A on node 0 (slot 0).
    gpus = [[0, 1], [0, 2]]
    ids = np.array([[0, 2], [2, 0], [1, 0]])
    assert eplb.remap(ids, gpus, 2).tolist() == [[0, 3], [3, 2], [1, 0]]


# ---- the library's native planner (host code: runs without a GPU) against the oracle

def _native():
    from expert_routing_grouped_amd import moe
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("library not built")
    return moe


def _check_native(moe, load, groups, nodes, gpus, phys, hier):
    p2l, offs, slots = moe.moe_eplb_place(load, groups, nodes, gpus, phys, hier)
    ref = np.array([e for g in eplb.place(load, groups, nodes, gpus, phys, hier) for e in g])
    assert np.array_equal(p2l, ref)
    E = len(load)
    for e in range(E):   # the replica table lists exactly the slots holding e, ascending
        assert np.array_equal(slots[offs[e]:offs[e + 1]], np.nonzero(ref == e)[0])
    assert offs[-1] == phys


def test_native_planner_matches_oracle_on_the_page_cases(page_sim):
    moe = _native()
    g, _, load = page_sim
    for c in g["cases"]:
        _check_native(moe, load, g["inputs"]["num_groups"], c["nodes"], c["gpus"], c["physical"],
                      c["strategy"] == "hierarchical")


@pytest.mark.parametrize("seed", range(6))
def test_native_planner_matches_oracle_on_random_loads(seed):
    moe = _native()
    rng = np.random.default_rng(seed)
    E, groups = [(64, 8), (96, 12), (256, 8)][seed % 3]
    # integer loads (many ties) or float loads, some zero
    load = rng.integers(0, 6, E).astype(float) if seed % 2 else rng.random(E) ** 3
    load[rng.integers(0, E, 4)] = 0.0
    for nodes, gpus, extra, hier in [(2, 8, 8, True), (4, 16, 16, True), (1, 4, 4, False),
                                     (4, 8, 8, False)]:
        if groups % nodes:
            continue
        _check_native(moe, load, groups, nodes, gpus, E + extra, hier)


def test_native_planner_validation():
    moe = _native()
    l = moe.lib()
    p = np.zeros(16, dtype=np.int32).ctypes.data_as(__import__("ctypes").c_void_p)
    load = np.ones(16).ctypes.data_as(__import__("ctypes").c_void_p)
    assert l.moe_eplb_place(load, 16, 4, 2, 4, 15, 1, p, p, p) == 1     # fewer slots than experts
    assert l.moe_eplb_place(load, 16, 3, 1, 4, 16, 0, p, p, p) == 1     # 3 does not divide 16
    assert l.moe_eplb_place(load, 16, 4, 3, 3, 18, 1, p, p, p) == 1     # 4 groups on 3 nodes
    assert l.moe_eplb_place(load, 16, 4, 2, 4, 18, 0, p, p, p) == 1     # 18 slots on 4 GPUs
    assert l.moe_eplb_place(None, 16, 4, 2, 4, 16, 1, p, p, p) == 1
    bad = np.ones(16)
    bad[3] = np.nan
    assert l.moe_eplb_place(bad.ctypes.data_as(__import__("ctypes").c_void_p), 16, 4, 2, 4, 16, 1,
                            p, p, p) == 1
