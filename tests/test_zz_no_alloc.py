"""moe_expert_ffn_noalloc (the allocation-free variant of moe_expert_ffn, on the library's fixed
scratch) against moe_expert_ffn on the same inputs, through the C ABI: two calls in a row on each
shape, the second with fewer tokens, so that the second runs on scratch that holds the first
call's h and partial sums. Same kernels, so the rows must be bit-identical (within 2e-2 of
max |o| is the bar for bf16 outputs; equality is stronger)."""
import numpy as np
import pytest

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


def _ffn_both(wl, T):
    """Route and dispatch T tokens of workload wl, then both FFN entry points on the result."""
    w = wl.replace(T=T)
    inp = W.generate(w)
    print(f"noalloc {wl.name} T={T} local={w.num_local} I={w.inter}", flush=True)
    scores = to_device(inp.scores, DEV)
    x = to_device(inp.x, DEV)
    wgu, wd = to_device(inp.w_gate_up, DEV), to_device(inp.w_down, DEV)
    ids, _ = moe.moe_route(scores, w.top_k, w.num_groups, w.topk_groups)
    d = moe.moe_dispatch(ids, w.expert_begin, w.num_local)
    cap = T * w.top_k
    ref = moe.moe_expert_ffn(x, d["offsets"], wgu, wd, row_index=d["sorted_assign"],
                             row_index_div=w.top_k, row_capacity=cap)
    out = torch.full((cap, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    moe.moe_expert_ffn_noalloc(x, d["offsets"], wgu, wd, out, row_index=d["sorted_assign"],
                               row_index_div=w.top_k, row_capacity=cap)
    torch.cuda.synchronize()
    M = int(to_host(d["offsets"])[-1])
    return to_host(ref)[:M], to_host(out)[:M], M


@pytest.mark.parametrize("name,T1,T2", [("decode_tp", 512, 97), ("decode_ep", 512, 40)])
def test_noalloc_matches_workspace_entry_point(name, T1, T2):
    wl = W.WORKLOADS[name]
    for T in (T1, T2):
        ref, got, M = _ffn_both(wl, T)
        assert M > 0
        assert np.array_equal(got, ref), f"{name} T={T}: rows differ"


def test_noalloc_refuses_sizes_beyond_the_scratch():
    """32768 rows x I = 2048 need 128 MiB of h: refused on the host, nothing enqueued."""
    rows, d, I = 32768, 256, 2048
    x = torch.zeros((rows, d), dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(2, dtype=torch.int32, device=DEV)
    wgu = torch.zeros((1, 2 * I, d), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((1, d, I), dtype=torch.bfloat16, device=DEV)
    o = torch.zeros_like(x)
    assert moe.ffn_workspace_size(1, d, I, rows, torch.bfloat16) > moe.NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError, match="fixed scratch"):
        moe.moe_expert_ffn_noalloc(x, offs, wgu, wd, o, row_capacity=rows)
