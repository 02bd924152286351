"""Pins of the oracle's "defer to a second round" and "send to a same-weight replica" overflow
policies (CH15 section 4.3, table of overflow policies; section 4.4, expert replication). CPU only."""
import numpy as np
import pytest

import oracle

# 5 tokens, k = 2, local experts 0..2 (3 is another GPU's). Assignment a = 2 t + j:
#   a0 t0 e0   a1 t0 e1   a2 t1 e0   a3 t1 e2   a4 t2 e1
#   a5 t2 e0   a6 t3 e0   a7 t3 e3   a8 t4 e2   a9 t4 e1
IDS = np.array([[0, 1], [0, 2], [1, 0], [0, 3], [2, 1]], np.int32)


def test_deferred_hand_example():
    # C = 2, two rounds. Ranks per expert: e0: a0 a2 a5 a6, e1: a1 a4 a9, e2: a3 a8.
    # Round 0 takes ranks 0, 1; round 1 ranks 2, 3.
    counts, offsets, sa, pos, demand = oracle.dispatch_deferred(IDS, 0, 3, 2, 2)
    assert counts.tolist() == [[2, 2, 2], [2, 1, 0]]
    assert offsets.tolist() == [[0, 2, 4, 6], [6, 8, 9, 9]]
    assert sa.tolist() == [0, 2, 1, 4, 3, 8, 5, 6, 9]
    assert pos.tolist() == [0, 2, 1, 4, 3, 6, 7, -1, 5, 8]
    assert demand.tolist() == [4, 3, 2]
    # one round: the drop policy; C = 1 with two rounds drops e0's ranks 2 and 3, e1's rank 2
    c1, o1, sa1, p1, _ = oracle.dispatch_deferred(IDS, 0, 3, 1, 2)
    assert c1.tolist() == [[1, 1, 1], [1, 1, 1]]
    assert sa1.tolist() == [0, 1, 3, 2, 4, 8]
    assert p1.tolist() == [0, 1, 3, 2, 4, -1, -1, -1, 5, -1]
    c0, o0, sa0, p0, d0 = oracle.dispatch_deferred(IDS, 0, 3, 0, 3)
    assert c0.sum() == 0 and sa0.size == 0 and (p0 == -1).all() and d0.tolist() == [4, 3, 2]


def _random_ids(rng, T, k, E):
    # distinct experts per token, skewed so that caps bite
    p = rng.dirichlet(np.full(E, 0.3))
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("seed,T,k,E,begin,nloc,C", [(0, 200, 4, 16, 0, 16, 9), (1, 300, 6, 24, 5, 10, 4),
                                                       (2, 50, 2, 8, 0, 8, 1)])
def test_deferred_one_round_is_the_drop_policy(seed, T, k, E, begin, nloc, C):
    ids = _random_ids(np.random.default_rng(seed), T, k, E)
    counts, offsets, sa, pos, demand = oracle.dispatch_deferred(ids, begin, nloc, C, 1)
    rc, ro, rsa, rpos, rdem = oracle.dispatch_capacity(ids, begin, nloc, C)
    assert np.array_equal(counts[0], rc) and np.array_equal(offsets[0], ro)
    assert np.array_equal(sa, rsa) and np.array_equal(pos, rpos) and np.array_equal(demand, rdem)


@pytest.mark.parametrize("seed,C,R", [(3, 5, 4), (4, 2, 3), (5, 7, 2)])
def test_deferred_rounds_structure_and_enough_rounds_lose_nothing(seed, C, R):
    rng = np.random.default_rng(seed)
    T, k, E, nloc = 120, 4, 12, 12
    ids = _random_ids(rng, T, k, E)
    counts, offsets, sa, pos, demand = oracle.dispatch_deferred(ids, 0, nloc, C, R)
    flat = ids.reshape(-1)
    assert (counts <= C).all()
    assert np.array_equal(counts.sum(0), np.minimum(demand, R * C))
    for r in range(R):
        for e in range(nloc):
            mine = np.flatnonzero(flat == e)                       # e's assignments in order
            rows = sa[offsets[r, e]:offsets[r, e + 1]]
            assert np.array_equal(rows, mine[r * C:(r + 1) * C])   # ranks [rC, (r+1)C)
        if r + 1 < R:
            assert offsets[r, nloc] == offsets[r + 1, 0]
    # with rounds enough for the busiest expert nothing is dropped, and the layer's output is
    # the dropless one (the same rows through the same experts, combined in slot order; up to
    # the last bits of the float64 matrix products, whose blocking follows the row count)
    R2 = int(-(-demand.max() // C))
    c2, o2, sa2, p2, _ = oracle.dispatch_deferred(ids, 0, nloc, C, R2)
    assert (p2 >= 0).all()
    d, I = 16, 8
    x = rng.standard_normal((T, d))
    wgu = rng.standard_normal((nloc, 2 * I, d)) / 4
    wd = rng.standard_normal((nloc, d, I)) / 4
    w = rng.random((T, k))
    o_rounds = np.zeros((sa2.size, d))
    for r in range(R2):                                           # one FFN call per round
        rows = slice(o2[r, 0], o2[r, nloc])
        o_rounds[rows] = oracle.expert_ffn(oracle.gather_rows(x, sa2, k)[rows], o2[r] - o2[r, 0], wgu, wd)
    y_rounds = oracle.combine(o_rounds, p2, w)
    _, off_d, sa_d, pos_d = oracle.dispatch(ids, 0, nloc)
    y_drop = oracle.combine(oracle.expert_ffn(oracle.gather_rows(x, sa_d, k), off_d, wgu, wd), pos_d, w)
    assert np.abs(y_rounds - y_drop).max() <= 1e-12 * np.abs(y_drop).max()
    assert np.array_equal(y_rounds == 0, y_drop == 0)


def test_replica_hand_example():
    # logical e0 has replicas [5, 2] (in that order), e1 one replica [0], e2 none; C = 1.
    # e0: a0 -> 5, a2 -> 2, a5, a6 -> -1; e1: a1 -> 0, a4, a9 -> -1; e2: a3, a8 -> -1;
    # a7 (expert 3) is outside [0, 3) -> -1.
    off = np.array([0, 2, 3, 3], np.int32)
    slots = np.array([5, 2, 0], np.int32)
    phys = oracle.remap_capacity(IDS, off, slots, 1)
    assert phys.tolist() == [[5, 0], [2, -1], [-1, -1], [-1, -1], [-1, -1]]
    # C = 2: e0's first two to replica 5, the next two to replica 2; e1's first two to 0
    phys2 = oracle.remap_capacity(IDS, off, slots, 2)
    assert phys2.tolist() == [[5, 0], [5, -1], [0, 2], [2, -1], [-1, -1]]
    assert (oracle.remap_capacity(IDS, off, slots, 0) == -1).all()


@pytest.mark.parametrize("seed,C", [(0, 3), (1, 10), (2, 1)])
def test_replica_properties(seed, C):
    rng = np.random.default_rng(seed)
    T, k, E = 150, 4, 16
    ids = _random_ids(rng, T, k, E)
    nrep = rng.integers(0, 4, size=E)
    off = np.concatenate([[0], np.cumsum(nrep)]).astype(np.int32)
    slots = rng.permutation(int(off[-1])).astype(np.int32)       # any order of physical slots
    phys = oracle.remap_capacity(ids, off, slots, C)
    flat, pf = ids.reshape(-1), phys.reshape(-1)
    owner = np.repeat(np.arange(E), nrep)                         # logical expert of each slot index
    live = pf >= 0
    assert np.array_equal(owner[np.argsort(slots)][pf[live]], flat[live])   # a replica of the same expert
    load = np.bincount(pf[live], minlength=int(off[-1]))
    assert (load <= C).all()
    demand = np.bincount(flat, minlength=E)
    assert live.sum() == np.minimum(demand, nrep * C).sum()
    # with one replica per expert the kept slots are exactly the drop policy's
    one = np.arange(E + 1, dtype=np.int32)
    p1 = oracle.remap_capacity(ids, one, np.arange(E, dtype=np.int32), C)
    _, _, _, pos, _ = oracle.dispatch_capacity(ids, 0, E, C)
    assert np.array_equal(p1.reshape(-1) >= 0, pos >= 0)
    # room for everything: every slot goes to its expert's first replica
    big = oracle.remap_capacity(ids, off, slots, T * k)
    has = nrep[flat] > 0
    assert np.array_equal(big.reshape(-1)[has], slots[off[flat[has]]])
    assert (big.reshape(-1)[~has] == -1).all()
