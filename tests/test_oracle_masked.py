"""Pins of the oracle's masked (fixed per-expert slot) layout: the dispatch into slots of C rows
per local expert with the drop policy (CH15 section 4.3, capacity factor; INFRA page, H20
paragraph: the masked grouped GEMM), and the expert FFN over the valid rows of each slot block.

CPU only."""
import numpy as np
import pytest

import oracle


def test_hand_example():
    # 4 tokens, k = 2, experts 0..2 all local, C = 2: expert 0 is asked by a = 0, 2, 5, 6 and keeps
    # 0, 2 in rows 0, 1; expert 1 by a = 1, 4, 7 keeps 1, 4 in rows 2, 3; expert 2 by a = 3 -> row 4
    ids = np.array([[0, 1], [0, 2], [1, 0], [0, 1]], dtype=np.int32)
    counts, slot_assign, pos, demand = oracle.dispatch_masked(ids, 0, 3, 2)
    assert counts.tolist() == [2, 2, 1]
    assert demand.tolist() == [4, 3, 1]
    assert slot_assign.tolist() == [0, 2, 1, 4, 3, -1]
    assert pos.tolist() == [0, 2, 1, 4, 3, -1, -1, -1]


@pytest.mark.parametrize("seed,T,k,E,begin,nloc,C", [
    (0, 64, 4, 16, 0, 16, 3), (1, 200, 8, 64, 8, 24, 10), (2, 37, 2, 8, 2, 3, 1),
    (3, 100, 8, 32, 0, 32, 1000), (4, 50, 3, 12, 0, 12, 0)])
def test_same_kept_rows_as_the_capped_dispatch(seed, T, k, E, begin, nloc, C):
    """The masked layout keeps exactly the rows of the capped dispatch, each expert's rows at the
    start of its own slot block instead of at a prefix-sum offset; empty slots are -1."""
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, slot_assign, pos, demand = oracle.dispatch_masked(ids, begin, nloc, C)
    c2, off, sa, pos2, d2 = oracle.dispatch_capacity(ids, begin, nloc, C)
    assert np.array_equal(counts, c2) and np.array_equal(demand, d2)
    for e in range(nloc):
        block = slot_assign[e * C:(e + 1) * C]
        assert np.array_equal(block[:counts[e]], sa[off[e]:off[e + 1]])
        assert (block[counts[e]:] == -1).all()
    # assign_pos is the inverse map: slot rows for kept assignments, -1 for the others
    kept = pos >= 0
    assert np.array_equal(kept, pos2 >= 0)
    assert np.array_equal(slot_assign[pos[kept]], np.nonzero(kept)[0])


def test_ffn_masked_equals_the_grouped_ffn_on_the_valid_rows():
    rng = np.random.default_rng(7)
    E_loc, C, d, I = 3, 4, 16, 8
    counts = np.array([2, 0, 4], dtype=np.int32)
    x_slots = rng.standard_normal((E_loc * C, d))
    x_slots[2:4] = 1e6          # padding of expert 0: must not reach any output
    wgu = rng.standard_normal((E_loc, 2 * I, d)) * 0.1
    wd = rng.standard_normal((E_loc, d, I)) * 0.1
    o = oracle.expert_ffn_masked(x_slots, counts, C, wgu, wd)
    rows = np.concatenate([np.arange(e * C, e * C + counts[e]) for e in range(E_loc)])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    ref = oracle.expert_ffn(x_slots[rows], offsets, wgu, wd)
    assert np.array_equal(o[rows], ref)
    others = np.setdiff1d(np.arange(E_loc * C), rows)
    assert (o[others] == 0).all()
    # counts above C are clamped to the block
    o2 = oracle.expert_ffn_masked(x_slots, np.array([9, 0, 4]), C, wgu, wd)
    assert np.array_equal(o2[0:4], oracle.expert_ffn(x_slots[0:4], np.array([0, 4, 4, 4]), wgu, wd)[0:4])
