"""Pins of the oracle's dispatch, expert FFN and combine (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from expert_routing_grouped_amd import workloads as W


# ---------------------------------------------------------------- dispatch

def _check_dispatch_properties(ids, begin, n_loc, counts, offsets, sorted_assign, assign_pos):
    """Properties that together fix a stable counting sort uniquely."""
    flat = ids.reshape(-1).astype(np.int64)
    local = [a for a in range(flat.size) if begin <= flat[a] < begin + n_loc]
    # counts by direct counting, offsets are their running sum
    for e in range(n_loc):
        assert counts[e] == sum(1 for a in local if flat[a] - begin == e)
    assert offsets[0] == 0
    assert all(offsets[e + 1] - offsets[e] == counts[e] for e in range(n_loc))
    # sorted_assign is a permutation of the local assignments ...
    assert sorted(sorted_assign.tolist()) == local
    # ... grouped by expert in the offsets' ranges, and increasing within an expert
    for e in range(n_loc):
        seg = sorted_assign[offsets[e]:offsets[e + 1]].tolist()
        assert all(flat[a] - begin == e for a in seg)
        assert seg == sorted(seg)
    # assign_pos is its inverse, -1 elsewhere
    for a in range(flat.size):
        if begin <= flat[a] < begin + n_loc:
            assert sorted_assign[assign_pos[a]] == a
        else:
            assert assign_pos[a] == -1


@pytest.mark.parametrize("T,k,E,begin,n_loc", [
    (40, 2, 8, 0, 8), (37, 4, 32, 8, 8), (64, 8, 256, 32, 32), (1, 1, 4, 0, 4), (50, 3, 16, 5, 3)])
def test_dispatch_properties(T, k, E, begin, n_loc):
    rng = np.random.default_rng(T + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    out = oracle.dispatch(ids, begin, n_loc)
    _check_dispatch_properties(ids, begin, n_loc, *out)


def test_dispatch_no_local_hit_and_empty():
    ids = np.full((5, 2), 9, dtype=np.int32)
    counts, offsets, sa, pos = oracle.dispatch(ids, 0, 4)
    assert counts.tolist() == [0] * 4 and offsets.tolist() == [0] * 5 and sa.size == 0
    assert (pos == -1).all()
    counts, offsets, sa, pos = oracle.dispatch(np.zeros((0, 2), np.int32), 0, 4)
    assert offsets.tolist() == [0] * 5 and sa.size == 0 and pos.size == 0


def test_dispatch_hand_example():
    # tokens: t0 -> (2, 0), t1 -> (0, 1), t2 -> (2, 1); assignments a = 2 t + j
    ids = np.array([[2, 0], [0, 1], [2, 1]], np.int32)
    counts, offsets, sa, pos = oracle.dispatch(ids, 0, 3)
    assert counts.tolist() == [2, 2, 2]
    assert offsets.tolist() == [0, 2, 4, 6]
    assert sa.tolist() == [1, 2, 3, 5, 0, 4]
    assert pos.tolist() == [4, 0, 1, 2, 5, 3]


# ---------------------------------------------------------------- expert FFN

def _one(x, wg, wu, wd):
    wgu = np.concatenate([np.asarray(wg, float), np.asarray(wu, float)])[None]
    xs = np.asarray(x, float)[None]
    return oracle.expert_ffn(xs, np.array([0, 1]), wgu, np.asarray(wd, float)[None])[0]


def test_silu_closed_forms():
    # silu(2) = 2 sigma(2) = 1 + tanh(1); 2 silu(1) = 2 sigma(1) * 2 / 2 ... = 1 + tanh(1/2)
    np.testing.assert_allclose(_one([1.0], [[2.0]], [[1.0]], [[1.0]]), [1 + math.tanh(1.0)], rtol=1e-14)
    # gate and up are not interchangeable: gate 1, up 2 gives 2 silu(1) = 1 + tanh(1/2)
    np.testing.assert_allclose(_one([1.0], [[1.0]], [[2.0]], [[1.0]]), [1 + math.tanh(0.5)], rtol=1e-14)
    # large negative gate saturates to zero without NaN
    out = _one([1.0], [[-1000.0]], [[3.0]], [[1.0]])
    assert np.isfinite(out).all() and out[0] == 0.0


def test_permutation_weights_closed_form():
    """Cyclic permutation matrices make every output a single product with known value.

    x = (a, b, c) = (1, 2, -1); gate = (b, c, a); up = (c, a, b);
    h = (silu(b) c, silu(c) a, silu(a) b); down reverses: o = (silu(a) b, silu(c) a, silu(b) c).
    With sigma(z) = (1 + tanh(z/2)) / 2:
    silu(1) * 2 = 1 + tanh(1/2); silu(-1) * 1 = -(1 - tanh(1/2)) / 2; silu(2) * -1 = -(1 + tanh(1)).
    A transposed matrix, a swapped gate/up or an index slip changes the result.
    """
    wg = [[0, 1, 0], [0, 0, 1], [1, 0, 0]]
    wu = [[0, 0, 1], [1, 0, 0], [0, 1, 0]]
    wd = [[0, 0, 1], [0, 1, 0], [1, 0, 0]]
    out = _one([1.0, 2.0, -1.0], wg, wu, wd)
    expect = [1 + math.tanh(0.5), -(1 - math.tanh(0.5)) / 2, -(1 + math.tanh(1.0))]
    np.testing.assert_allclose(out, expect, rtol=1e-14)


def test_ffn_zero_and_linear_cases():
    rng = np.random.default_rng(3)
    E_loc, d, I, M = 3, 8, 6, 7
    wgu = rng.standard_normal((E_loc, 2 * I, d))
    wd = rng.standard_normal((E_loc, d, I))
    offsets = np.array([0, 3, 3, 7])                      # expert 1 has no rows
    x = rng.standard_normal((M, d))
    o = oracle.expert_ffn(x, offsets, wgu, wd)
    # x = 0 gives 0
    assert not oracle.expert_ffn(np.zeros_like(x), offsets, wgu, wd).any()
    # up projection 0 gives 0
    wz = wgu.copy()
    wz[:, I:] = 0
    assert not oracle.expert_ffn(x, offsets, wz, wd).any()
    # linear in the down projection and in the up projection
    np.testing.assert_allclose(oracle.expert_ffn(x, offsets, wgu, 3 * wd), 3 * o, rtol=1e-12)
    wu3 = wgu.copy()
    wu3[:, I:] *= -2
    np.testing.assert_allclose(oracle.expert_ffn(x, offsets, wu3, wd), -2 * o, rtol=1e-12)
    # rows are independent: any subset computed alone matches
    rows = np.array([6, 0, 4])
    sub = oracle.expert_ffn_rows(x[rows], np.array([2, 0, 2]), wgu, wd)
    np.testing.assert_allclose(sub, o[rows], rtol=1e-13)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3E80, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[:5].tolist() == [1.0, -2.0, 0.0, -0.0, 0.25]
    assert math.copysign(1, vals[3]) == -1
    assert vals[5] == (2 - 2 ** -7) * 2.0 ** 127
    assert vals[6] == 2.0 ** -133
    # the generator's rounding is to nearest even
    f = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert oracle.bf16_bits_to_f64(W.f32_to_bf16_bits(f)).tolist() == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7]


# ---------------------------------------------------------------- combine and layer

def test_combine_closed_forms():
    o = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    # token 0 slots -> rows 2 and 0; token 1 only slot 1 local (row 1); token 2 none
    pos = np.array([2, 0, -1, 1, -1, -1])
    w = np.array([[0.5, 0.25], [0.9, 0.75], [1.0, 1.0]])
    y = oracle.combine(o, pos, w)
    np.testing.assert_allclose(y, [[50.25, 100.5], [7.5, 15.0], [0.0, 0.0]], rtol=1e-15)


def _dense_per_token(x, ids, w, wgu, wd, begin, n_loc):
    """Dense per-token FFN with plain loops, no permutation: y[t] = sum_j w[t,j] FFN_e(x[t])."""
    T, k = ids.shape
    I = wgu.shape[1] // 2
    d = wgu.shape[2]
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j]) - begin
            if not 0 <= e < n_loc:
                continue
            h = []
            for i in range(I):
                g = sum(wgu[e, i, c] * x[t, c] for c in range(d))
                u = sum(wgu[e, I + i, c] * x[t, c] for c in range(d))
                h.append(g / (1 + math.exp(-g)) * u)
            for c in range(d):
                y[t, c] += w[t, j] * sum(wd[e, c, i] * h[i] for i in range(I))
    return y


@pytest.mark.parametrize("begin,n_loc", [(0, 8), (2, 3)])
def test_layer_matches_dense_per_token(begin, n_loc):
    rng = np.random.default_rng(11)
    T, E, k, d, I = 9, 8, 2, 5, 3
    scores = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d))
    wgu = rng.standard_normal((n_loc, 2 * I, d)) * 0.5
    wd = rng.standard_normal((n_loc, d, I)) * 0.5
    out = oracle.layer(scores, x, wgu, wd, top_k=k, num_groups=1, topk_groups=1,
                       score_mode="softmax", renormalize=False, expert_begin=begin, num_local=n_loc)
    dense = _dense_per_token(x, out["topk_ids"], out["topk_weights"], wgu, wd, begin, n_loc)
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-14)


def test_identical_experts_weights_sum_to_one():
    """All experts equal and renormalised weights: y = FFN(x) for every token."""
    rng = np.random.default_rng(4)
    T, E, d, I = 6, 16, 4, 3
    scores = rng.random((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d))
    wgu1 = rng.standard_normal((2 * I, d))
    wd1 = rng.standard_normal((d, I))
    wgu = np.repeat(wgu1[None], E, 0)
    wd = np.repeat(wd1[None], E, 0)
    out = oracle.layer(scores, x, wgu, wd, top_k=4, num_groups=4, topk_groups=2, score_mode="raw",
                       renormalize=True, expert_begin=0, num_local=E)
    single = oracle.expert_ffn(x, np.array([0, T]), wgu1[None], wd1[None])
    np.testing.assert_allclose(out["y"], single, rtol=1e-12)
