"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: routing ids, counts, offsets, permutation and gathered rows bit-exact;
float32 outputs max|err| / max|ref| <= 1e-4; bf16 outputs <= 2e-2.
"""
import json
import os

import numpy as np
import pytest

import oracle
from expert_routing_grouped_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from expert_routing_grouped_amd import moe  # noqa: E402
from expert_routing_grouped_amd.tensors import to_device, to_host  # noqa: E402

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda:0"


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max() if ref.size else 0.0
    if scale == 0.0:
        return float(np.abs(got).max()) if got.size else 0.0
    return float(np.abs(got - ref).max() / scale)


def as_f64(a):
    a = np.asarray(a)
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.fixture(scope="module", autouse=True)
def _gpu(gpu):
    moe.lib()
    yield


_CACHE = {}


def inputs(name, with_ffn=True):
    key = (name, with_ffn)
    if key not in _CACHE:
        _CACHE.clear() if with_ffn and name.startswith("prefill") else None
        _CACHE[key] = W.generate(W.WORKLOADS[name], with_ffn=with_ffn)
    return _CACHE[key]


def gpu_route(scores, k, ng, tg, mode, renorm):
    s = to_device(np.ascontiguousarray(scores, dtype=np.float32), DEV)
    ids, w = moe.moe_route(s, k, ng, tg, mode, renorm)
    torch.cuda.synchronize()
    return to_host(ids), to_host(w)


def oracle_route(scores, k, ng, tg, mode, renorm):
    if mode == moe.MOE_SCORE_SOFTMAX:
        return oracle.route_softmax_topk(scores, k, renorm)
    return oracle.route_grouped(scores, k, ng, tg, renorm)


def check_route(scores, k, ng, tg, mode=moe.MOE_SCORE_RAW, renorm=True):
    print(f"route T={scores.shape[0]} E={scores.shape[1]} k={k} groups={ng}/{tg} mode={mode}", flush=True)
    ids, w = gpu_route(scores, k, ng, tg, mode, renorm)
    rids, rw = oracle_route(scores, k, ng, tg, mode, renorm)
    assert np.array_equal(ids, rids)
    assert rel_err(w, rw) <= TOL_F32
    return ids, w


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("name", ["route_permute", "decode_ep", "prefill_straggler"])
def test_route_workloads(name):
    wl = W.WORKLOADS[name]
    check_route(inputs(name, with_ffn=False).scores, wl.top_k, wl.num_groups, wl.topk_groups)


def test_route_toy_softmax():
    wl = W.WORKLOADS["toy_fp32"]
    s = inputs("toy_fp32", with_ffn=False).scores
    check_route(s, wl.top_k, 1, 1, moe.MOE_SCORE_SOFTMAX, False)
    check_route(s, wl.top_k, 1, 1, moe.MOE_SCORE_SOFTMAX, True)


def test_route_page_simulation_reproduces_printed_numbers():
    g = json.load(open(os.path.join(GOLDEN, "page_eplb_no_eplb.json")))
    p = g["inputs"]
    s = W.page_simulation_scores(T=p["T"], E=p["E"], seed=p["seed"])
    ids, _ = check_route(s, p["top_k"], p["num_groups"], p["topk_groups"])
    load = np.bincount(ids.ravel(), minlength=p["E"]).astype(float)
    for case in g["cases"]:
        gl = load.reshape(case["gpus"], -1).sum(axis=1)
        assert f"{gl.max() / gl.mean():.2f}" == case["busiest_over_mean"]


@pytest.mark.parametrize("E,ng,tg,k", [(64, 8, 4, 8), (256, 8, 4, 8), (256, 1, 1, 8), (16, 4, 2, 3)])
def test_route_tie_stress(E, ng, tg, k):
    check_route(W.tie_stress_scores(500, E, seed=E + k), k, ng, tg, renorm=False)


def test_route_handcrafted_golden():
    g = json.load(open(os.path.join(GOLDEN, "router_handcrafted.json")))
    for case in g["cases"]:
        s = np.array([case["scores"]], dtype=np.float32)
        ids, w = gpu_route(s, case["top_k"], g["num_groups"], case["topk_groups"],
                           moe.MOE_SCORE_RAW, case["renormalize"])
        assert ids[0].tolist() == case["ids"], case["name"]
        np.testing.assert_allclose(w[0], case["weights"], rtol=1e-6, atol=0)


@pytest.mark.parametrize("E,ng,tg,k,mode", [
    (96, 8, 3, 6, moe.MOE_SCORE_RAW),      # 12 experts per group over 2-wide lanes: general group path
    (896, 1, 1, 16, moe.MOE_SCORE_RAW),    # 896 experts, 16 per token, no groups
    (1024, 64, 8, 16, moe.MOE_SCORE_RAW),  # many small groups
    (8, 1, 1, 2, moe.MOE_SCORE_SOFTMAX),
    (40, 1, 1, 40, moe.MOE_SCORE_SOFTMAX), # every expert selected
    (300, 10, 4, 12, moe.MOE_SCORE_RAW),   # E not a multiple of 64
])
def test_route_shapes(E, ng, tg, k, mode):
    rng = np.random.default_rng(E)
    s = (rng.random((333, E)) + 0.15 * rng.normal(0, 1, E)).astype(np.float32)
    check_route(s, k, ng, tg, mode, renorm=True)


def test_route_empty():
    s = torch.empty((0, 256), dtype=torch.float32, device=DEV)
    ids, w = moe.moe_route(s, 8, 8, 4)
    torch.cuda.synchronize()
    assert ids.shape == (0, 8)


# ------------------------------------------------------------------ dispatch

def check_dispatch(ids, begin, nloc, x=None):
    k = ids.shape[1]
    print(f"dispatch T={ids.shape[0]} k={k} local=[{begin},{begin + nloc}) x={x is not None}", flush=True)
    d_ids = to_device(np.ascontiguousarray(ids, dtype=np.int32), DEV)
    d_x = to_device(x, DEV) if x is not None else None
    out = moe.moe_dispatch(d_ids, begin, nloc, d_x)
    torch.cuda.synchronize()
    counts, offsets, sa, pos = oracle.dispatch(ids, begin, nloc)
    M = int(offsets[-1])
    assert np.array_equal(to_host(out["counts"]), counts)
    assert np.array_equal(to_host(out["offsets"]), offsets)
    assert np.array_equal(to_host(out["sorted_assign"])[:M], sa)
    assert np.array_equal(to_host(out["assign_pos"])[:ids.size], pos)
    if x is not None:
        xs = to_host(out["x_sorted"])[:M]
        assert np.array_equal(xs, oracle.gather_rows(x, sa, k))
    return out


@pytest.mark.parametrize("name,begin,nloc", [
    ("route_permute", 0, 256), ("route_permute", 0, 8), ("route_permute", 32, 32),
    ("route_permute", 100, 17), ("prefill_straggler", 32, 32), ("prefill_straggler", 0, 256)])
def test_dispatch_workloads(name, begin, nloc):
    wl = W.WORKLOADS[name]
    ids, _ = oracle.route_grouped(inputs(name, with_ffn=False).scores, wl.top_k, wl.num_groups,
                                  wl.topk_groups)
    check_dispatch(ids, begin, nloc)


@pytest.mark.parametrize("T,k,E,begin,nloc", [
    (1, 1, 4, 0, 4), (37, 3, 16, 3, 5), (1000, 8, 64, 0, 64), (513, 8, 1000, 0, 1000),
    (513, 8, 1024, 0, 1024), (1100, 8, 1030, 3, 1024),
    (5, 2, 8, 6, 2), (4096, 2, 2, 0, 1),
    # above 8192 assignments: the multi-workgroup sort, ragged last block, and
    # beyond 256 blocks of 2048 where each block's share grows
    (1100, 8, 1000, 0, 1000), (8193, 1, 3, 0, 3), (70001, 8, 256, 5, 200)])
def test_dispatch_ragged(T, k, E, begin, nloc):
    rng = np.random.default_rng(T * 7 + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, 64)).astype(np.float32)
    check_dispatch(ids, begin, nloc, x)


def test_dispatch_no_local_hit_and_empty():
    ids = np.full((64, 4), 200, dtype=np.int32)
    ids[:, 1:] = np.arange(201, 204)
    out = check_dispatch(ids, 0, 8)
    assert (to_host(out["assign_pos"]) == -1).all()
    d_ids = torch.empty((0, 8), dtype=torch.int32, device=DEV)
    o = moe.moe_dispatch(d_ids, 0, 8)
    torch.cuda.synchronize()
    assert (to_host(o["offsets"]) == 0).all() and (to_host(o["counts"]) == 0).all()


def test_dispatch_gathers_bf16_rows():
    inp = inputs("decode_ep")
    wl = inp.workload
    ids, _ = oracle.route_grouped(inp.scores, wl.top_k, wl.num_groups, wl.topk_groups)
    check_dispatch(ids, wl.expert_begin, wl.num_local, inp.x)


# ------------------------------------------------------------------ full layer

def run_layer(inp, wl, fuse=True):
    """The four calls on the GPU; returns host copies of every output.

    fuse: the FFN reads token rows through sorted_assign (gather fused into GEMM-1);
    otherwise moe_dispatch materialises x_sorted and the FFN reads that."""
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    layer = moe.MoELayer(num_tokens=wl.T, num_experts=wl.E, top_k=wl.top_k,
                         num_groups=wl.num_groups, topk_groups=wl.topk_groups,
                         score_mode=moe.MOE_SCORE_SOFTMAX if wl.score_mode == "softmax" else moe.MOE_SCORE_RAW,
                         renormalize=wl.renormalize, expert_begin=wl.expert_begin,
                         num_local_experts=wl.num_local, hidden=wl.hidden, inter=wl.inter,
                         dtype=dt, device=DEV, fuse_gather=fuse)
    s, x = to_device(inp.scores, DEV), to_device(inp.x, DEV)
    wgu, wd = to_device(inp.w_gate_up, DEV), to_device(inp.w_down, DEV)
    print(f"layer {wl.name} T={wl.T} d={wl.hidden} I={wl.inter} local={wl.num_local} fuse={fuse}",
          flush=True)
    layer.forward(s, x, wgu, wd)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in layer.buf.items() if k != "workspace"}


def oracle_front(inp, wl):
    ids, w = oracle.route(inp.scores, wl.top_k, wl.num_groups, wl.topk_groups, wl.score_mode,
                          wl.renormalize)
    counts, offsets, sa, pos = oracle.dispatch(ids, wl.expert_begin, wl.num_local)
    return ids, w, counts, offsets, sa, pos


def check_front(g, ref):
    ids, w, counts, offsets, sa, pos = ref
    M = int(offsets[-1])
    assert np.array_equal(g["topk_ids"], ids)
    assert rel_err(g["topk_weights"], w) <= TOL_F32
    assert np.array_equal(g["counts"], counts) and np.array_equal(g["offsets"], offsets)
    assert np.array_equal(g["sorted_assign"][:M], sa)
    assert np.array_equal(g["assign_pos"][:ids.size], pos)
    return M


def small_bf16_workload(T, E, k, ng, tg, d, I, begin, nloc, seed):
    return W.Workload(f"small_{T}_{E}_{d}_{I}", T=T, E=E, top_k=k, num_groups=ng, topk_groups=tg,
                      score_mode="raw", renormalize=True, bias_std=1.0, hidden=d, inter=I,
                      expert_begin=begin, num_local=nloc, dtype="bf16", seed=seed)


def check_full(wl, inp, tol, fuse=True):
    g = run_layer(inp, wl, fuse)
    ref = oracle_front(inp, wl)
    M = check_front(g, ref)
    ids, w, counts, offsets, sa, pos = ref
    xs = oracle.gather_rows(inp.x, sa, wl.top_k)
    if not fuse:
        assert np.array_equal(g["x_sorted"][:M], xs)
    o_ref = oracle.expert_ffn(xs, offsets, inp.w_gate_up, inp.w_down)
    e_o = rel_err(as_f64(g["o_sorted"][:M]), o_ref)
    y_ref = oracle.combine(o_ref, pos, w)
    e_y = rel_err(as_f64(g["y"]), y_ref)
    print(f"  M={M} rel_err o={e_o:.3e} y={e_y:.3e}", flush=True)
    assert e_o <= tol and e_y <= tol
    # tokens with no local slot get exact zero rows
    none_local = (pos.reshape(wl.T, wl.top_k) < 0).all(axis=1)
    assert not as_f64(g["y"])[none_local].any()
    return g


@pytest.mark.parametrize("fuse", [True, False])
def test_layer_toy_fp32(fuse):
    wl = W.WORKLOADS["toy_fp32"]
    check_full(wl, inputs("toy_fp32"), TOL_F32, fuse)


@pytest.mark.parametrize("T,E,k,ng,tg,d,I,begin,nloc", [
    (96, 16, 4, 4, 2, 512, 128, 0, 16),     # several row tiles per expert, ragged tails
    (300, 32, 8, 8, 4, 256, 64, 4, 12),     # local range in the middle, I = 64
    (40, 64, 6, 8, 4, 1024, 192, 0, 64),    # many experts with 0-9 rows
    (700, 8, 2, 1, 1, 256, 256, 0, 8),      # > 64 rows per expert
    (1200, 4, 2, 1, 1, 512, 128, 0, 4),     # > 256 rows per expert: 128 x 128 tiles, ragged
    (1500, 4, 2, 1, 1, 2048, 1024, 0, 4),   # 128 x 128 tiles, K = 2048
    (2100, 16, 8, 2, 1, 512, 256, 0, 16),   # row capacity >= 16384 but 160 large tiles (< 3/4 of the CUs): 128 x 128
    (2100, 16, 8, 2, 1, 512, 192, 2, 12),   # same capacity, I % 128 != 0: 128 x 128 tiles
    (2060, 16, 8, 4, 2, 4096, 512, 0, 16),  # >= one 256 x 256 tile per CU in both GEMMs, ragged
    (2048, 64, 8, 1, 1, 2048, 1024, 0, 4),  # experts of 589, 69, 70, 376 rows, row capacity 16384
    # narrow experts: shared activation tiles, K split in 2 / 1 / 4 parts + finalize
    (300, 32, 8, 8, 4, 2048, 64, 4, 12),
    (200, 16, 4, 4, 2, 1024, 128, 0, 16),
    (700, 8, 2, 1, 1, 4096, 128, 0, 8),
    (1200, 4, 2, 1, 1, 1024, 64, 0, 4),     # > 256 rows per expert, all in 64-row chunks
])
@pytest.mark.parametrize("fuse", [True, False])
def test_layer_bf16_small(T, E, k, ng, tg, d, I, begin, nloc, fuse):
    wl = small_bf16_workload(T, E, k, ng, tg, d, I, begin, nloc, seed=T + d)
    check_full(wl, W.generate(wl), TOL_BF16, fuse)


@pytest.mark.parametrize("fuse", [True, False])
def test_layer_decode_ep_full(fuse):
    wl = W.WORKLOADS["decode_ep"]
    check_full(wl, inputs("decode_ep"), TOL_BF16, fuse)


def test_layer_decode_tp_full_and_deterministic():
    wl = W.WORKLOADS["decode_tp"]
    inp = inputs("decode_tp")
    g1 = check_full(wl, inp, TOL_BF16)
    g2 = run_layer(inp, wl)
    for key in ("topk_ids", "topk_weights", "sorted_assign", "y"):
        assert np.array_equal(g1[key], g2[key]), key


@pytest.mark.parametrize("name", ["prefill_straggler", "prefill_literal"])
def test_layer_prefill_sampled(name):
    """Full-size prefill share: routing and permutation exact; o and y checked on sampled rows."""
    wl = W.WORKLOADS[name]
    inp = inputs(name)
    g = run_layer(inp, wl)
    ref = oracle_front(inp, wl)
    M = check_front(g, ref)
    ids, w, counts, offsets, sa, pos = ref
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(M, size=min(M, 192), replace=False),
                                     offsets[1:][counts > 0] - 1]))   # includes every expert's last row
    local_e = np.searchsorted(offsets, rows, side="right") - 1
    toks = rng.choice(wl.T, size=48, replace=False)
    pairs = [(i, t, j, int(pos[t * wl.top_k + j])) for i, t in enumerate(toks)
             for j in range(wl.top_k) if pos[t * wl.top_k + j] >= 0]
    pair_e = np.array([np.searchsorted(offsets, p, side="right") - 1 for *_, p in pairs], dtype=np.int64)
    # one oracle call for the sampled rows and for every local slot of the sampled tokens
    x_rows = np.concatenate([inp.x[sa[rows] // wl.top_k], inp.x[[t for _, t, _, _ in pairs]]])
    o_all = oracle.expert_ffn_rows(x_rows, np.concatenate([local_e, pair_e]), inp.w_gate_up,
                                   inp.w_down)
    o_ref = o_all[:rows.size]
    e_o = rel_err(as_f64(g["o_sorted"][rows]), o_ref)
    y_ref = np.zeros((toks.size, wl.hidden))
    for q, (i, t, j, _) in enumerate(pairs):          # slot order within each token
        y_ref[i] += w[t, j] * o_all[rows.size + q]
    e_y = rel_err(as_f64(g["y"][toks]), y_ref)
    print(f"  M={M} sampled rows={rows.size} rel_err o={e_o:.3e} y={e_y:.3e}", flush=True)
    assert e_o <= TOL_BF16 and e_y <= TOL_BF16


def test_layer_prefill_straggler_every_row():
    """The prefill_straggler share at full size (d = 7168, I = 2048, 14312 rows, both GEMMs on
    the large-tile kernel for the 10 experts above 64 rows and the streaming kernel for the
    other 6): every row of o and every token of y against the float64 oracle."""
    name = "prefill_straggler"
    wl = W.WORKLOADS[name]
    inp = inputs(name)
    g = run_layer(inp, wl)
    ref = oracle_front(inp, wl)
    M = check_front(g, ref)
    ids, w, counts, offsets, sa, pos = ref
    o_ref = oracle.expert_ffn(oracle.gather_rows(inp.x, sa, wl.top_k), offsets, inp.w_gate_up, inp.w_down)
    e_o = rel_err(as_f64(g["o_sorted"][:M]), o_ref)
    y_ref = oracle.combine(o_ref, pos, w)
    del o_ref
    e_y = rel_err(as_f64(g["y"]), y_ref)
    print(f"  M={M} every row: rel_err o={e_o:.3e} y={e_y:.3e}", flush=True)
    assert e_o <= TOL_BF16 and e_y <= TOL_BF16


def test_layer_prefill_routing_every_row():
    """The prefill_straggler routing (experts of 2 .. 2659 rows) at d = 2048, I = 2048: the
    large-tile kernel runs both GEMMs and takes every expert above 64 rows (the ones with 97
    and 102 rows as single partly filled tiles), the streaming kernel the rest; every row of
    o and y is checked against the oracle."""
    wl = W.WORKLOADS["prefill_straggler"].replace(name="prefill_straggler_d2048", hidden=2048)
    check_full(wl, W.generate(wl), TOL_BF16)


def test_layer_prefill_literal_routing_every_row():
    """The prefill_literal routing (5 experts of 87 .. 506 rows above 64, two below) at d = 2048,
    I = 2048: 7 large tiles per column block, 112 items per GEMM, too few for the large-tile
    kernel, so both GEMMs take 128 x 128 tiles (at d = 7168 the down GEMM's 196 items take the
    large tiles: test_layer_prefill_sampled); every row of o and y against the oracle, and a
    second run bit-identical to the first."""
    wl = W.WORKLOADS["prefill_literal"].replace(name="prefill_literal_d2048", hidden=2048)
    inp = W.generate(wl)
    g1 = check_full(wl, inp, TOL_BF16)
    g2 = run_layer(inp, wl)
    for key in ("o_sorted", "y"):
        assert np.array_equal(g1[key], g2[key]), key


# ------------------------------------------------------------------ capacity-limited dispatch

def check_dispatch_capacity(ids, begin, nloc, cap, x=None):
    k = ids.shape[1]
    print(f"dispatch_capacity T={ids.shape[0]} k={k} local=[{begin},{begin + nloc}) C={cap}", flush=True)
    d_ids = to_device(np.ascontiguousarray(ids, dtype=np.int32), DEV)
    d_x = to_device(x, DEV) if x is not None else None
    out = moe.moe_dispatch(d_ids, begin, nloc, d_x, capacity=cap)
    torch.cuda.synchronize()
    counts, offsets, sa, pos, demand = oracle.dispatch_capacity(ids, begin, nloc, cap)
    M = int(offsets[-1])
    assert np.array_equal(to_host(out["counts"]), counts)
    assert np.array_equal(to_host(out["offsets"]), offsets)
    assert np.array_equal(to_host(out["demand"]), demand)
    assert np.array_equal(to_host(out["sorted_assign"])[:M], sa)
    assert np.array_equal(to_host(out["assign_pos"])[:ids.size], pos)
    if x is not None:
        assert np.array_equal(to_host(out["x_sorted"])[:M], oracle.gather_rows(x, sa, k))
    return out


def test_dispatch_capacity_workload():
    """The capacity-factor example of ch15 section 4.3 (T = 5600, k = 16 of E = 896, C = 120):
    routing then the capped dispatch, bit-exact against the oracle."""
    wl = W.WORKLOADS["capacity_route"]
    scores = inputs("capacity_route", with_ffn=False).scores
    ids, _ = oracle.route(scores, wl.top_k, 1, 1, "raw", True)
    d_ids, _ = moe.moe_route(to_device(scores, DEV), wl.top_k, 1, 1, moe.MOE_SCORE_RAW, True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d_ids), ids)
    cap = oracle.expert_capacity(wl.T, wl.top_k, wl.E, wl.capacity_factor)
    out = check_dispatch_capacity(ids, 0, wl.E, cap)
    assert (to_host(out["demand"]) > cap).any()


@pytest.mark.parametrize("T,k,E,begin,nloc,cap", [
    (40, 4, 16, 0, 16, 3),           # single-workgroup sort
    (500, 8, 64, 5, 40, 50),
    (300, 6, 20, 0, 20, 0),          # everything dropped
    (300, 6, 20, 0, 20, 10 ** 6),    # nothing dropped: equals moe_dispatch
    (3000, 8, 300, 0, 300, 70),      # multi-workgroup sort
    (70001, 8, 256, 5, 200, 2000),   # beyond 256 blocks
    (9000, 2, 4, 1, 2, 1)])
def test_dispatch_capacity_ragged(T, k, E, begin, nloc, cap):
    rng = np.random.default_rng(T + cap)
    # skewed expert choice, so that caps bite
    p = rng.random(E) ** 4
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, 32)).astype(np.float32) if T <= 3000 else None
    check_dispatch_capacity(ids, begin, nloc, cap, x)
    if cap >= T * k:
        check_dispatch(ids, begin, nloc)


def test_layer_with_capacity_drops_contributions():
    """Capped dispatch feeding the FFN and combine: dropped slots contribute nothing."""
    wl = small_bf16_workload(400, 16, 4, 4, 2, 512, 128, 0, 16, seed=11)
    inp = W.generate(wl)
    ids, w = oracle.route(inp.scores, wl.top_k, wl.num_groups, wl.topk_groups, "raw", True)
    cap = 40
    layer = moe.MoELayer(num_tokens=wl.T, num_experts=wl.E, top_k=wl.top_k, num_groups=wl.num_groups,
                         topk_groups=wl.topk_groups, score_mode=moe.MOE_SCORE_RAW, renormalize=True,
                         expert_begin=0, num_local_experts=wl.num_local, hidden=wl.hidden,
                         inter=wl.inter, dtype=torch.bfloat16, device=DEV, expert_capacity=cap)
    y = layer.forward(to_device(inp.scores, DEV), to_device(inp.x, DEV), to_device(inp.w_gate_up, DEV),
                      to_device(inp.w_down, DEV))
    torch.cuda.synchronize()
    counts, offsets, sa, pos, demand = oracle.dispatch_capacity(ids, 0, wl.num_local, cap)
    assert (demand > cap).any()
    assert np.array_equal(to_host(layer.buf["assign_pos"])[:ids.size], pos)
    o_ref = oracle.expert_ffn(oracle.gather_rows(inp.x, sa, wl.top_k), offsets, inp.w_gate_up, inp.w_down)
    y_ref = oracle.combine(o_ref, pos, w)
    assert rel_err(as_f64(to_host(y)), y_ref) <= TOL_BF16


# ------------------------------------------------------------------ EPLB replica choice

@pytest.mark.parametrize("nodes,gpus,phys,hier", [(4, 32, 288, False), (4, 32, 288, True),
                                                  (8, 64, 320, False), (8, 64, 320, True),
                                                  (1, 8, 256, False)])
def test_eplb_remap_matches_oracle(nodes, gpus, phys, hier):
    """Placement of the EPLB page's simulation (native planner), then the GPU replica choice for
    all 20000 routed tokens against the oracle; the first 2000 tokens reproduce the page's
    printed nodes-per-token figure."""
    from oracle import eplb
    scores = W.page_simulation_scores()
    ids, _ = oracle.route_grouped(scores, 8, 8, 4)
    load = np.bincount(ids.ravel(), minlength=256).astype(float)
    p2l, offs, slots = moe.moe_eplb_place(load, 8, nodes, gpus, phys, hier)
    print(f"eplb remap nodes={nodes} gpus={gpus} phys={phys} hier={hier}", flush=True)
    got = moe.moe_eplb_remap(to_device(ids, DEV), to_device(offs, DEV), to_device(slots, DEV), gpus, nodes)
    torch.cuda.synchronize()
    gpus_list = [p2l[g * (phys // gpus):(g + 1) * (phys // gpus)].tolist() for g in range(gpus)]
    ref = eplb.remap(ids, gpus_list, nodes)
    assert np.array_equal(to_host(got), ref)
    assert np.array_equal(p2l[to_host(got)], ids)


def test_eplb_remap_out_of_range_ids_get_minus_one():
    """Expert ids outside [0, E) and experts without a replica map to -1; the other slots of the
    same token keep the oracle's choice (the invalid slots add no node)."""
    from oracle import eplb
    rng = np.random.default_rng(5)
    E, gpus, nodes, phys = 16, 4, 2, 16
    load = rng.integers(1, 50, E).astype(float)
    p2l, offs, slots = moe.moe_eplb_place(load, 4, nodes, gpus, phys, False)
    ids = np.stack([rng.choice(E, size=4, replace=False) for _ in range(256)]).astype(np.int32)
    bad = ids.copy()
    bad[::3, 1] = E + 7
    bad[1::5, 2] = -3
    bad[2::7, 0] = 1 << 30
    print("eplb remap with invalid ids", flush=True)
    got = to_host(moe.moe_eplb_remap(to_device(bad, DEV), to_device(offs, DEV), to_device(slots, DEV),
                                     gpus, nodes))
    valid = (bad >= 0) & (bad < E)
    assert (got[~valid] == -1).all()
    gpus_list = [p2l[g * (phys // gpus):(g + 1) * (phys // gpus)].tolist() for g in range(gpus)]
    for t in range(bad.shape[0]):   # the valid slots of each token, alone, through the oracle
        keep = valid[t]
        ref = eplb.remap(bad[t:t + 1, keep], gpus_list, nodes)
        assert np.array_equal(got[t, keep], ref[0])
    # an expert with no replica: a table where expert 0's range is empty
    offs2 = offs.copy()
    offs2[0] = offs2[1]
    got2 = to_host(moe.moe_eplb_remap(to_device(ids, DEV), to_device(offs2, DEV), to_device(slots, DEV),
                                      gpus, nodes))
    assert (got2[ids == 0] == -1).all()
