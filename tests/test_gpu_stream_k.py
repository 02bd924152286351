"""The gate_up GEMM of narrow experts (inter <= 128) on the stream-K kernel.

The K steps of all (chunk, 64-column slab) pairs are shared out over the grid,
so a pair can be split over several workgroups: the pieces of a split pair
write float32 partial sums into the workspace (the first piece also a record
of its pair), and ffn_finalize_kernel adds the pieces in K order. Nothing may
depend on what the workspace held before the call, so the same call is made
on workspaces filled with zero bytes, 0xFF bytes and random bytes and on a buffer that served the previous
call: every output must be the same bit for bit and within the bf16 bar (2e-2
of max|ref|) of the float64 oracle. The cases split pairs in two or three
pieces, over many workgroups, and a single chunk over the whole grid.
"""
import numpy as np
import pytest

import oracle
from expert_routing_grouped_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from expert_routing_grouped_amd import moe  # noqa: E402
from expert_routing_grouped_amd.tensors import to_device, to_host  # noqa: E402

DEV = "cuda:0"
TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu(gpu):
    moe.lib()
    yield


def rel_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / scale)


# (name, T, E, k, groups, local, d, I): 256 narrow experts with about 16 rows each (pairs split in
# two or three pieces); four experts with many rows and two slabs (few pairs, each split over
# many workgroups); one expert with every token (a single chunk spread over the grid).
CASES = [
    ("narrow256", 512, 256, 8, 8, 256, 2048, 64),
    ("few_wide", 96, 8, 2, 1, 4, 1024, 128),
    ("one_expert", 300, 4, 1, 1, 1, 1024, 64),
]


@pytest.mark.parametrize("name,T,E,k,ng,nloc,d,I", CASES, ids=[c[0] for c in CASES])
def test_stream_k_workspace_contents(name, T, E, k, ng, nloc, d, I):
    wl = W.Workload(name, T=T, E=E, top_k=k, num_groups=ng, topk_groups=max(1, ng // 2),
                    score_mode="raw", renormalize=True, bias_std=1.0, hidden=d, inter=I,
                    expert_begin=0, num_local=nloc, dtype="bf16", seed=5)
    print(f"stream-K {name}: T={T} E={E} k={k} local={nloc} d={d} I={I}", flush=True)
    inp = W.generate(wl)
    ids, w = oracle.route(inp.scores, k, wl.num_groups, wl.topk_groups, "raw", True)
    counts, offsets, sa, pos = oracle.dispatch(ids, 0, nloc)
    M = int(offsets[-1])
    assert M > 0
    x = to_device(inp.x, DEV)
    off = to_device(offsets.astype(np.int32), DEV)
    cap = T * k
    ri_host = np.zeros(cap, dtype=np.int32)    # rows past M are never read
    ri_host[:M] = sa[:M]
    ri = to_device(ri_host, DEV)
    wgu, wd = to_device(inp.w_gate_up, DEV), to_device(inp.w_down, DEV)
    need = moe.ffn_workspace_size(nloc, d, I, cap, torch.bfloat16)
    gen = torch.Generator(device=DEV).manual_seed(3)
    fills = {
        "zeros": torch.zeros(need, dtype=torch.uint8, device=DEV),
        "ones": torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV),
        "random": torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=gen),
    }
    outs = {}
    for key, ws in fills.items():
        outs[key] = to_host(moe.moe_expert_ffn(x, off, wgu, wd, row_index=ri, row_index_div=k,
                                               row_capacity=cap, workspace=ws))[:M]
        torch.cuda.synchronize()
    # the buffer of the last call again, twice (its flags were cleared by that call)
    ws = fills["random"]
    for rep in range(2):
        outs[f"reuse{rep}"] = to_host(moe.moe_expert_ffn(x, off, wgu, wd, row_index=ri, row_index_div=k,
                                                         row_capacity=cap, workspace=ws))[:M]
        torch.cuda.synchronize()
    base = outs["zeros"]
    for key, o in outs.items():
        assert np.array_equal(o, base), key
    o_ref = oracle.expert_ffn(oracle.gather_rows(inp.x, sa, k), offsets, inp.w_gate_up, inp.w_down)
    e = rel_err(oracle.bf16_bits_to_f64(base), o_ref)
    print(f"  M={M} rel_err o={e:.3e}", flush=True)
    assert e <= TOL_BF16
