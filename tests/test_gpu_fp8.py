"""GPU parity of the FP8 path (moe_quantize_e4m3, moe_expert_ffn_fp8) against oracle/fp8.py.

Bars: the quantiser's codes and scales bit-exact (both sides decide in
float32 from the same float32 values); the FFN's float32 h within 1e-4 of
max|h| of the oracle's float64 h (the float32 bar); the FFN's own quantisation of h bit-exact
against the oracle's quantiser applied to the kernel's h; o and y (bf16)
within 2e-2 of max|ref|, with a mean error below 2e-3 of it.
"""
import numpy as np
import pytest

import oracle
from oracle import fp8 as F
from expert_routing_grouped_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from expert_routing_grouped_amd import moe  # noqa: E402
from expert_routing_grouped_amd.tensors import to_device, to_host  # noqa: E402

DEV = "cuda:0"
TOL_H = 1e-4
TOL_O = 2e-2
TOL_O_MEAN = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu(gpu):
    moe.lib()
    yield


def bf16_f64(a):
    return oracle.bf16_bits_to_f64(a)


def errs(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    d = np.abs(got - ref)
    return float(d.max() / scale), float(d.mean() / scale)


# ------------------------------------------------------------------ quantiser

def _rows(rng, R, C):
    x = (rng.standard_normal((R, C)) * rng.uniform(1e-3, 30.0, (R, 1))).astype(np.float32)
    if R > 2:
        x[1, :128] = 0.0                                    # an all-zero block
        x[2, 128:256] = rng.uniform(-1, 1, 128) * 2.0 ** -12 if C > 128 else x[2, 128:256]
        # a block whose amax is 448: scale exactly 1, so midpoints between e4m3 values are ties
        pos = F.e4m3_positive_values()
        mids = (pos[:-1] + pos[1:]) / 2                      # 126 ties
        x[0, :128] = np.concatenate([[448.0], mids, [1.0]]) * np.where(np.arange(128) % 2, -1, 1)
    return x


@pytest.mark.parametrize("R,C", [(1, 128), (37, 256), (513, 7168), (4, 2048)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_bit_exact(R, C, dtype):
    print(f"quantize R={R} C={C} {dtype}", flush=True)
    rng = np.random.default_rng(R * 7 + C)
    x = _rows(rng, R, C)
    if dtype == "bf16":
        bits = W.f32_to_bf16_bits(x)
        x = bf16_f64(bits).astype(np.float32)
        xd = to_device(bits, DEV)
    else:
        xd = to_device(x, DEV)
    codes, scales = moe.moe_quantize_e4m3(xd)
    torch.cuda.synchronize()
    rc, rs = F.quantize_rows(x)
    assert np.array_equal(to_host(codes), rc)
    assert np.array_equal(to_host(scales).view(np.uint32), rs.view(np.uint32))


def test_quantize_e4m3_rounding_dense():
    """Every 128-value block holds +-448, so its scale is exactly 1 and the codes are the plain e4m3
    rounding of the other 127 values: for each interval between neighbouring e4m3 values its ends,
    the midpoint (a tie), the float32 values one ulp either side of those, and random interior
    values; also values below the smallest subnormal, both signs. Codes and scales bit-exact
    against the oracle's table-based encoder."""
    rng = np.random.default_rng(4481)
    pos = F.e4m3_positive_values().astype(np.float32)
    vals = [np.float32(0.0), np.float32(2.0 ** -11), np.float32(2.0 ** -10), np.float32(3 * 2.0 ** -11)]
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = np.float32((np.float64(lo) + np.float64(hi)) / 2)
        for v in (lo, hi, mid):
            vals += [v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))]
        vals += list(rng.uniform(lo, hi, 4).astype(np.float32))
    v = np.abs(np.array(vals, dtype=np.float32))
    v = v[v <= 448.0]
    v = np.concatenate([v, -v])
    rng.shuffle(v)
    nb = (v.size + 126) // 127
    v = np.concatenate([v, np.zeros(nb * 127 - v.size, np.float32)]).reshape(nb, 127)
    blocks = np.concatenate([np.where(np.arange(nb)[:, None] % 2, -448.0, 448.0).astype(np.float32), v], axis=1)
    x = blocks.reshape(-1, 8 * 128) if nb % 8 == 0 else \
        np.concatenate([blocks, np.tile(blocks[:1], (8 - nb % 8, 1))]).reshape(-1, 8 * 128)
    print(f"dense e4m3 rounding: {x.size} values in {x.shape[0]} rows", flush=True)
    codes, scales = moe.moe_quantize_e4m3(to_device(x, DEV))
    torch.cuda.synchronize()
    rc, rs = F.quantize_rows(x)
    assert (rs == 1.0).all()
    assert np.array_equal(to_host(codes), rc)
    assert np.array_equal(to_host(codes).reshape(-1), F.e4m3_encode(x.reshape(-1)))
    assert np.array_equal(to_host(scales).view(np.uint32), rs.view(np.uint32))


def test_quantize_no_rows():
    x = torch.zeros((0, 256), dtype=torch.float32, device=DEV)
    c, s = moe.moe_quantize_e4m3(x)
    torch.cuda.synchronize()
    assert c.shape == (0, 256) and s.shape == (0, 2)


# ------------------------------------------------------------------ FFN

def fp8_weights(rng, nloc, d, I, scale=0.05, distinct=None):
    """E4M3 weights with 128 x 128 block scales; with `distinct`, that many random experts
    repeated in turn (cheap inputs for many local experts)."""
    n = nloc if distinct is None else distinct
    wgu = (rng.standard_normal((n, 2 * I, d)) * scale).astype(np.float32)
    wd = (rng.standard_normal((n, d, I)) * scale).astype(np.float32)
    out = W.quantize_e4m3_blocks(wgu, 128) + W.quantize_e4m3_blocks(wd, 128)
    if n == nloc:
        return out
    idx = np.arange(nloc) % n
    return tuple(np.ascontiguousarray(a[idx]) for a in out)


SENTINEL = 0x7FC1   # a bf16 NaN pattern that no output row holds


def run_ffn(xq, xs, sa, k, offsets, wts, I, cap):
    wgq, wgs, wdq, wds = wts
    nloc, d = wgq.shape[0], wgq.shape[2]
    dev = lambda a: to_device(np.ascontiguousarray(a), DEV)
    ri = None if sa is None else dev(np.asarray(sa, np.int32))
    need = moe.ffn_fp8_workspace_size(nloc, d, I, cap)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o_buf = dev(np.full((cap, d), SENTINEL, np.uint16))
    if sa is not None:   # token rows: pad the row index to the capacity
        ri = dev(np.concatenate([np.asarray(sa, np.int32), np.zeros(max(0, cap - len(sa)), np.int32)]))
    o = moe.moe_expert_ffn_fp8(dev(xq), dev(xs), dev(np.asarray(offsets, np.int32)), dev(wgq), dev(wgs),
                               dev(wdq), dev(wds), row_index=ri, row_index_div=k, row_capacity=cap,
                               o_sorted=o_buf, workspace=ws)
    torch.cuda.synchronize()
    # The workspace holds h (float32, [cap, I]), then its codes and scales, each
    # region 256-byte aligned.
    a256 = lambda n: (n + 255) // 256 * 256
    wsh = to_host(ws)
    h = wsh[:cap * I * 4].view(np.float32).reshape(cap, I)
    o1 = a256(cap * I * 4)
    hq = wsh[o1:o1 + cap * I].reshape(cap, I)
    o2 = o1 + a256(cap * I)
    hs = wsh[o2:o2 + cap * (I // 128) * 4].view(np.float32).reshape(cap, I // 128)
    return to_host(o), h, hq, hs


def check_ffn(counts, d, I, k, seed, permuted=False, spare_rows=0, distinct=None):
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts)
    nloc, M = counts.size, int(counts.sum())
    offsets = np.concatenate([[0], np.cumsum(counts)])
    T = max(1, -(-M // k) + 3)
    x = rng.standard_normal((T, d)).astype(np.float32)
    xq, xs = F.quantize_rows(x)
    sa = rng.permutation(T * k)[:M]                     # distinct assignments t * k + j
    wts = fp8_weights(rng, nloc, d, I, distinct=distinct)
    print(f"ffn_fp8 experts={nloc} rows={M} d={d} I={I} k={k} permuted={permuted} spare={spare_rows}",
          flush=True)
    cap = max(M, 1) + spare_rows
    if permuted:      # x given as permuted rows (row_index NULL)
        rows = np.concatenate([sa // k, np.zeros(cap - M, np.int64)])
        g_o, g_h, g_hq, g_hs = run_ffn(xq[rows], xs[rows], None, 1, offsets, wts, I, cap)
    else:
        g_o, g_h, g_hq, g_hs = run_ffn(xq, xs, sa, k, offsets, wts, I, cap)
    o, hq, hs = F.expert_ffn_fp8(xq, xs, sa, k, offsets, *wts, I)
    assert (g_o[M:] == SENTINEL).all()   # rows past offsets[E_loc] are not written
    if M == 0:
        return
    # h: float32 from the kernel's accumulation vs the oracle's float64
    wgq, wgs = wts[0], wts[1]
    h_ref = np.zeros((M, I))
    X = F.dequantize_rows(xq[sa // k], xs[sa // k])
    for e in range(nloc):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            W1 = F.dequantize_weights(wgq[e], wgs[e])
            g, u = X[lo:hi] @ W1[:I].T, X[lo:hi] @ W1[I:].T
            h_ref[lo:hi] = g / (1 + np.exp(-g)) * u
    e_h = np.abs(g_h[:M] - h_ref).max() / np.abs(h_ref).max()
    # the kernel's quantisation of its own h is the oracle's quantiser, bit for bit
    rq, rs = F.quantize_rows(g_h[:M])
    assert np.array_equal(g_hq[:M], rq) and np.array_equal(g_hs[:M].view(np.uint32), rs.view(np.uint32))
    same = (g_hq[:M] == hq).mean()
    e_o, m_o = errs(bf16_f64(g_o[:M]), o)
    print(f"  M={M} rel_err h={e_h:.2e} h codes equal={same:.5f} o={e_o:.2e} (mean {m_o:.2e})", flush=True)
    assert e_h <= TOL_H
    assert e_o <= TOL_O and m_o <= TOL_O_MEAN


@pytest.mark.parametrize("counts,d,I,k", [
    ([5, 0, 64, 1], 512, 256, 4),              # empty expert, exactly one chunk, one row
    ([65, 17, 130, 0, 3], 1024, 256, 2),       # several chunks with ragged tails
    ([33, 200], 2048, 512, 8),                  # K steps not a multiple of the pipeline period
    ([0, 0, 7], 512, 768, 3),                   # inter = 768: 3 h scale blocks per row
    ([300], 1536, 256, 1),                      # one expert, 5 chunks
])
def test_ffn_fp8_ragged(counts, d, I, k):
    check_ffn(counts, d, I, k, seed=sum(counts) + d + I)


# Experts with more than 64 rows take 128-row tiles (128 weight rows x 128 tokens per item).
@pytest.mark.parametrize("counts,d,I,k", [
    ([129, 0, 65, 64, 300, 1], 1024, 512, 4),   # 64 streamed / 65 tiled, a one-row last tile
    ([1000], 2048, 256, 8),                     # 8 tiles, the last with 104 rows
    ([128, 256, 200], 512, 768, 2),             # whole tiles; inter = 768: 12 gated N blocks
    ([70, 3, 190, 0, 0, 2500], 1536, 256, 8),   # a 20-tile expert beside streamed ones
])
def test_ffn_fp8_tiled(counts, d, I, k):
    check_ffn(counts, d, I, k, seed=sum(counts) * 3 + d + I)


def test_ffn_fp8_tiled_permuted_and_spare_rows():
    check_ffn([90, 0, 300], 1024, 512, 2, seed=13, permuted=True)
    check_ffn([90, 0, 300], 1024, 512, 2, seed=14, spare_rows=200)


def test_ffn_fp8_tiled_1024_local_experts():
    rng = np.random.default_rng(15)
    counts = rng.integers(0, 4, 1024) * (rng.random(1024) < 0.3)
    counts[[5, 400, 1023]] = [70, 300, 129]
    check_ffn(counts.tolist(), 512, 256, 8, seed=16, distinct=7)


# A prefill-sized row capacity (>= 16384) launches the 256 x 256 tile kernel too, which takes
# the experts above 64 rows when their tiles x N blocks fill 3/4 of the CUs (here 30 tiles x 8
# N blocks in both GEMMs); with fewer the 128-row tiles keep them.
BIG_CAP = 16384


@pytest.mark.parametrize("permuted", [False, True])
def test_ffn_fp8_large_tiles(permuted):
    counts = [1000, 0, 2600, 65, 300, 2050, 64, 1, 700]      # 30 tiles of 256, ragged last tiles
    M = sum(counts)
    check_ffn(counts, 2048, 1024, 8, seed=21 + permuted, spare_rows=BIG_CAP - M, permuted=permuted)


def test_ffn_fp8_large_capacity_no_rows():
    check_ffn([0, 0, 0, 0], 2048, 1024, 8, seed=24, spare_rows=BIG_CAP)   # both kernels find no work


def test_ffn_fp8_large_tiles_1024_local_experts():
    """1024 local experts at a prefill-sized capacity: the lists of both kernels span every
    expert, 30 of them large enough for 256-row tiles (4 tiles each is 120 x 8 N blocks)."""
    rng = np.random.default_rng(25)
    counts = rng.integers(0, 4, 1024) * (rng.random(1024) < 0.3)
    big = rng.choice(1024, 30, replace=False)
    counts[big] = rng.integers(769, 1025, 30)
    M = int(counts.sum())
    check_ffn(counts.tolist(), 512, 1024, 8, seed=26, distinct=5, spare_rows=max(0, BIG_CAP - M))


@pytest.mark.parametrize("seed", [31, 32, 33])
def test_ffn_fp8_large_tiles_random(seed):
    """Random expert sizes at a prefill-sized capacity: a skewed mix of empty, streamed (<= 64
    rows) and tiled experts, the 256-row tiles filling the GPU or not depending on the draw."""
    rng = np.random.default_rng(seed)
    nloc = int(rng.integers(8, 40))
    counts = (rng.pareto(1.2, nloc) * rng.uniform(40, 400)).astype(np.int64)
    counts[rng.random(nloc) < 0.2] = 0
    d, I = int(rng.choice([1024, 2048])), int(rng.choice([512, 1024]))
    M = int(counts.sum())
    check_ffn(counts.tolist(), d, I, 8, seed=seed + 100, spare_rows=max(0, BIG_CAP - M) + int(rng.integers(0, 50)))


def test_ffn_fp8_large_capacity_few_tiles():
    counts = [300, 0, 200, 40]                                 # 3 tiles of 256 x 8 N blocks: too few
    check_ffn(counts, 2048, 1024, 8, seed=23, spare_rows=BIG_CAP - sum(counts))


def test_ffn_fp8_permuted_rows():
    check_ffn([40, 0, 90], 1024, 512, 2, seed=3, permuted=True)


def test_ffn_fp8_no_rows():
    check_ffn([0, 0, 0], 512, 256, 2, seed=4)


def test_ffn_fp8_capacity_above_rows():
    check_ffn([20, 0, 45], 1024, 256, 4, seed=5, spare_rows=77)
    check_ffn([20, 0, 45], 1024, 256, 4, seed=6, spare_rows=77, permuted=True)


def test_ffn_fp8_1024_local_experts():
    rng = np.random.default_rng(8)
    counts = rng.integers(0, 4, 1024) * (rng.random(1024) < 0.3)
    check_ffn(counts.tolist(), 512, 256, 8, seed=9, distinct=7)


# ------------------------------------------------------------------ layer at the decode_ep_fp8 size

@pytest.mark.parametrize("name", ["decode_ep_fp8", "prefill_straggler_fp8"])
def test_layer_fp8_sampled(name):
    """Full-size FP8 shares through MoELayer (decode: every expert streamed; prefill: the
    straggler GPU's experts on 128-row tiles): routing and permutation exact, x's codes exact,
    o and y checked on sampled rows and tokens."""
    wl = W.WORKLOADS[name]
    inp = W.generate(wl)
    layer = moe.MoELayer(num_tokens=wl.T, num_experts=wl.E, top_k=wl.top_k, num_groups=wl.num_groups,
                         topk_groups=wl.topk_groups, score_mode=moe.MOE_SCORE_RAW,
                         renormalize=wl.renormalize, expert_begin=wl.expert_begin,
                         num_local_experts=wl.num_local, hidden=wl.hidden, inter=wl.inter,
                         dtype=torch.bfloat16, device=DEV, fp8=True)
    dev = lambda a: to_device(a, DEV)
    print(f"layer {wl.name} T={wl.T} d={wl.hidden} I={wl.inter} local={wl.num_local}", flush=True)
    layer.forward(dev(inp.scores), dev(inp.x), dev(inp.w_gate_up), dev(inp.w_down),
                  w_gate_up_scales=dev(inp.w_gate_up_scale), w_down_scales=dev(inp.w_down_scale))
    torch.cuda.synchronize()
    g = {k: to_host(v) for k, v in layer.buf.items() if k != "workspace"}
    # a second pass gives the same bits (no atomics, fixed summation order)
    y2 = to_host(layer.forward(dev(inp.scores), dev(inp.x), dev(inp.w_gate_up), dev(inp.w_down),
                               w_gate_up_scales=dev(inp.w_gate_up_scale),
                               w_down_scales=dev(inp.w_down_scale)))
    assert np.array_equal(y2, g["y"])
    ids, w = oracle.route(inp.scores, wl.top_k, wl.num_groups, wl.topk_groups, wl.score_mode,
                          wl.renormalize)
    counts, offsets, sa, pos = oracle.dispatch(ids, wl.expert_begin, wl.num_local)
    M = int(offsets[-1])
    assert np.array_equal(g["topk_ids"], ids)
    assert np.array_equal(g["offsets"], offsets) and np.array_equal(g["sorted_assign"][:M], sa)
    x32 = bf16_f64(inp.x).astype(np.float32)
    xq, xs = F.quantize_rows(x32)
    assert np.array_equal(g["x_codes"], xq) and np.array_equal(g["x_scales"], xs)
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(wl.T, size=24, replace=False))
    slots = [(t, j, int(pos[t * wl.top_k + j])) for t in toks for j in range(wl.top_k)
             if pos[t * wl.top_k + j] >= 0]
    rows = np.array([p for _, _, p in slots], np.int64)
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    # oracle on the sampled rows only: regroup them by expert
    order = np.argsort(e_of, kind="stable")
    sub_off = np.concatenate([[0], np.cumsum(np.bincount(e_of, minlength=wl.num_local))])
    o_sub, _, _ = F.expert_ffn_fp8(xq, xs, sa[rows[order]], wl.top_k, sub_off, inp.w_gate_up,
                                   inp.w_gate_up_scale, inp.w_down, inp.w_down_scale, wl.inter)
    o_ref = np.empty_like(o_sub)
    o_ref[order] = o_sub
    e_o, m_o = errs(bf16_f64(g["o_sorted"][rows]), o_ref)
    y_ref = np.zeros((toks.size, wl.hidden))
    ti = {t: i for i, t in enumerate(toks)}
    for q, (t, j, _) in enumerate(slots):
        y_ref[ti[t]] += float(w[t, j]) * o_ref[q]
    e_y, m_y = errs(bf16_f64(g["y"][toks]), y_ref)
    print(f"  M={M} sampled rows={rows.size} o={e_o:.2e} (mean {m_o:.2e}) y={e_y:.2e} (mean {m_y:.2e})",
          flush=True)
    assert e_o <= TOL_O and m_o <= TOL_O_MEAN and e_y <= TOL_O and m_y <= TOL_O_MEAN
