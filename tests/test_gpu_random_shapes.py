"""Seeded random shapes through the whole layer: the HIP path against the oracle.

Each case draws its sizes from a seed (tokens, experts, groups, k, the local
range, d, I, the activation form), runs route -> dispatch -> FFN -> combine on
the GPU through the C ABI and checks it with the same bars as the fixed cases:
routing, counts, offsets and permutation bit-exact; float32 outputs within 1e-4
and bf16 outputs within 2e-2 of max|ref|. FP8 cases check the FP8 FFN on the
routed rows (codes of x bit-exact, o within 2e-2 with a mean error below 2e-3).
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


@pytest.fixture(scope="module", autouse=True)
def _gpu(gpu):
    moe.lib()
    yield


def rel_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = np.abs(ref).max() if ref.size else 0.0
    return float(np.abs(got - ref).max() / scale) if scale > 0 else float(np.abs(got).max(initial=0.0))


def draw_shape(seed, dtype):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([8, 16, 32, 64, 128, 256]))
    groups = [g for g in (1, 2, 4, 8) if E % g == 0 and (g == 1 or E // g >= 2)]
    ng = int(rng.choice(groups))
    tg = int(rng.integers(1, ng + 1))
    k = int(rng.integers(1, min(8, tg * (E // ng)) + 1))
    T = int(rng.integers(1, 400))
    nloc = int(rng.integers(1, E + 1))
    begin = int(rng.integers(0, E - nloc + 1))
    if dtype == "f32":
        d, I = int(rng.choice([8, 64, 128, 264])), int(rng.choice([4, 32, 96, 128]))
    else:
        d, I = int(rng.choice([256, 512, 768, 1024, 2048])), int(rng.choice([64, 128, 192, 256, 512]))
    nloc = max(1, min(nloc, 60_000_000 // (3 * d * I)))   # bounded host-side weight draws
    begin = min(begin, E - nloc)
    return W.Workload(f"random{seed}", T=T, E=E, top_k=k, num_groups=ng, topk_groups=tg,
                      score_mode="raw", renormalize=bool(rng.integers(0, 2)),
                      bias_std=float(rng.choice([0.5, 1.0, 2.0])), hidden=d, inter=I,
                      expert_begin=begin, num_local=nloc, dtype=dtype, seed=seed), bool(rng.integers(0, 2))


def run_layer(wl, inp, fuse):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    layer = moe.MoELayer(num_tokens=wl.T, num_experts=wl.E, top_k=wl.top_k, num_groups=wl.num_groups,
                         topk_groups=wl.topk_groups, score_mode=moe.MOE_SCORE_RAW,
                         renormalize=wl.renormalize, expert_begin=wl.expert_begin,
                         num_local_experts=wl.num_local, hidden=wl.hidden, inter=wl.inter, dtype=dt,
                         device=DEV, fuse_gather=fuse)
    layer.forward(to_device(inp.scores, DEV), to_device(inp.x, DEV), to_device(inp.w_gate_up, DEV),
                  to_device(inp.w_down, DEV))
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in layer.buf.items() if k != "workspace"}


@pytest.mark.parametrize("seed,dtype", [(s, "bf16") for s in range(24)] + [(s, "f32") for s in range(8)])
def test_random_layer(seed, dtype):
    wl, fuse = draw_shape(seed, dtype)
    print(f"{wl.name} {dtype}: T={wl.T} E={wl.E} groups={wl.num_groups}/{wl.topk_groups} k={wl.top_k} "
          f"local=[{wl.expert_begin},{wl.expert_begin + wl.num_local}) d={wl.hidden} I={wl.inter} "
          f"renorm={wl.renormalize} fuse={fuse}", flush=True)
    inp = W.generate(wl)
    g = run_layer(wl, inp, fuse)
    ref = oracle.layer(inp.scores, inp.x, inp.w_gate_up, inp.w_down, top_k=wl.top_k,
                       num_groups=wl.num_groups, topk_groups=wl.topk_groups, score_mode="raw",
                       renormalize=wl.renormalize, expert_begin=wl.expert_begin, num_local=wl.num_local)
    M = int(ref["offsets"][-1])
    assert np.array_equal(g["topk_ids"], ref["topk_ids"])
    assert np.array_equal(g["counts"], ref["counts"]) and np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["sorted_assign"][:M], ref["sorted_assign"])
    assert np.array_equal(g["assign_pos"][:wl.T * wl.top_k], ref["assign_pos"])
    tol = 2e-2 if dtype == "bf16" else 1e-4
    dec = oracle.bf16_bits_to_f64 if dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    assert rel_err(g["topk_weights"], ref["topk_weights"]) <= 1e-4
    if M:
        e_o = rel_err(dec(g["o_sorted"][:M]), ref["o_sorted"])
        e_y = rel_err(dec(g["y"]), ref["y"])
        print(f"  M={M} rel_err o={e_o:.2e} y={e_y:.2e}", flush=True)
        assert e_o <= tol and e_y <= tol
    else:
        assert not dec(g["y"]).any()


@pytest.mark.parametrize("seed", range(8))
def test_random_fp8_ffn(seed):
    rng = np.random.default_rng(5000 + seed)
    d = int(rng.choice([512, 1024, 1536]))
    I = int(rng.choice([256, 512]))
    nloc = int(rng.integers(1, 40))
    k = int(rng.integers(1, 9))
    counts = rng.integers(0, 150, nloc) * (rng.random(nloc) < 0.7)
    M = int(counts.sum())
    T = max(1, -(-M // k) + int(rng.integers(0, 5)))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sa = rng.permutation(T * k)[:M].astype(np.int32)
    print(f"fp8 seed={seed}: experts={nloc} rows={M} T={T} k={k} d={d} I={I}", flush=True)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wgu = (rng.standard_normal((nloc, 2 * I, d)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((nloc, d, I)) * 0.05).astype(np.float32)
    wgq, wgs = W.quantize_e4m3_blocks(wgu, 128)
    wdq, wds = W.quantize_e4m3_blocks(wd, 128)
    dev = lambda a: to_device(np.ascontiguousarray(a), DEV)
    xq_d, xs_d = moe.moe_quantize_e4m3(dev(W.f32_to_bf16_bits(x)))
    cap = max(M, 1)
    ri = dev(np.concatenate([sa, np.zeros(cap - M, np.int32)]))
    o = moe.moe_expert_ffn_fp8(xq_d, xs_d, dev(offsets), dev(wgq), dev(wgs), dev(wdq), dev(wds),
                               row_index=ri, row_index_div=k, row_capacity=cap)
    torch.cuda.synchronize()
    xq, xs = F.quantize_rows(oracle.bf16_bits_to_f64(W.f32_to_bf16_bits(x)).astype(np.float32))
    assert np.array_equal(to_host(xq_d), xq) and np.array_equal(to_host(xs_d), xs)
    if M == 0:
        return
    ref, _, _ = F.expert_ffn_fp8(xq, xs, sa, k, offsets, wgq, wgs, wdq, wds, I)
    got = oracle.bf16_bits_to_f64(to_host(o)[:M])
    scale = np.abs(ref).max()
    e_max, e_mean = np.abs(got - ref).max() / scale, np.abs(got - ref).mean() / scale
    print(f"  rel_err o={e_max:.2e} (mean {e_mean:.2e})", flush=True)
    assert e_max <= 2e-2 and e_mean <= 2e-3


@pytest.mark.parametrize("d,I", [(256, 64), (1024, 64)])
def test_layer_1024_local_experts(d, I):
    """The largest local expert count of the whole layer (1024, the limit of every call):
    streaming path (d = 256) and the shared-activation path for narrow experts (d = 1024, I = 64)."""
    wl = W.Workload("local1024", T=512, E=1024, top_k=8, num_groups=8, topk_groups=4, score_mode="raw",
                    renormalize=True, bias_std=1.0, hidden=d, inter=I, expert_begin=0, num_local=1024,
                    dtype="bf16", seed=d + I)
    print(f"{wl.name}: T={wl.T} E={wl.E} local=1024 d={d} I={I}", flush=True)
    inp = W.generate(wl)
    g = run_layer(wl, inp, True)
    ref = oracle.layer(inp.scores, inp.x, inp.w_gate_up, inp.w_down, top_k=wl.top_k,
                       num_groups=wl.num_groups, topk_groups=wl.topk_groups, score_mode="raw",
                       renormalize=True, expert_begin=0, num_local=1024)
    M = int(ref["offsets"][-1])
    assert np.array_equal(g["topk_ids"], ref["topk_ids"])
    assert np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["sorted_assign"][:M], ref["sorted_assign"])
    e_o = rel_err(oracle.bf16_bits_to_f64(g["o_sorted"][:M]), ref["o_sorted"])
    e_y = rel_err(oracle.bf16_bits_to_f64(g["y"]), ref["y"])
    print(f"  M={M} hit={int((ref['counts'] > 0).sum())} rel_err o={e_o:.2e} y={e_y:.2e}", flush=True)
    assert e_o <= 2e-2 and e_y <= 2e-2
