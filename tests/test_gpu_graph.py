"""The layer's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The C ABI promises that its calls never synchronise the host and allocate
nothing, so a sequence of them can be captured. The graph is replayed several
times with eager work and synchronisations between the replays; every replay
must give the eager result bit for bit, also after the inputs are overwritten
in place.
"""
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


def _layer(wl, fp8=False):
    return moe.MoELayer(num_tokens=wl.T, num_experts=wl.E, top_k=wl.top_k, num_groups=wl.num_groups,
                        topk_groups=wl.topk_groups, score_mode=moe.MOE_SCORE_RAW,
                        renormalize=wl.renormalize, expert_begin=wl.expert_begin,
                        num_local_experts=wl.num_local, hidden=wl.hidden, inter=wl.inter,
                        dtype=torch.bfloat16, device=DEV, fp8=fp8)


# decode: streamed experts only; prefill: a row capacity of 65536 and about 24 k local rows, so the
# large-tile kernels take the experts above 64 rows (and, on FP8, quantise their rows of h);
# narrow: inter = 64, the stream-K gate_up kernel, whose split pairs pass partial sums through the
# workspace to the finalize kernel (bf16 only: the FP8 path needs inter to be a multiple of 128).
@pytest.mark.parametrize("size", ["decode", "prefill", "narrow"])
@pytest.mark.parametrize("fp8", [False, True])
def test_layer_graph_replays_match_eager(fp8, size):
    if fp8 and size == "narrow":
        pytest.skip("the FP8 FFN needs inter to be a multiple of 128")
    T, k, I = {"decode": (96, 6, 256), "prefill": (8192, 8, 512), "narrow": (256, 8, 64)}[size]
    wl = W.Workload("graph", T=T, E=64, top_k=k, num_groups=8, topk_groups=4, score_mode="raw",
                    renormalize=True, bias_std=1.0, hidden=1024, inter=I, expert_begin=8,
                    num_local=24, dtype="bf16", seed=11,
                    weight_format="fp8_e4m3_b128" if fp8 else "same")
    print(f"graph capture fp8={fp8} {size}: T={wl.T} E={wl.E} local={wl.num_local} d={wl.hidden} I={wl.inter}",
          flush=True)
    inp = W.generate(wl)
    inp2 = W.generate(wl.replace(seed=12))
    scores, x = to_device(inp.scores, DEV), to_device(inp.x, DEV)
    wgu, wd = to_device(inp.w_gate_up, DEV), to_device(inp.w_down, DEV)
    sc = dict(w_gate_up_scales=to_device(inp.w_gate_up_scale, DEV),
              w_down_scales=to_device(inp.w_down_scale, DEV)) if fp8 else {}

    eager = _layer(wl, fp8)
    y_ref = to_host(eager.forward(scores, x, wgu, wd, **sc))
    torch.cuda.synchronize()

    layer = _layer(wl, fp8)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # warm-up outside the capture (one-time queries)
        layer.forward(scores, x, wgu, wd, **sc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y = layer.forward(scores, x, wgu, wd, **sc)
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), y_ref), f"replay {rep}"
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        del junk

    # new inputs written in place: the replay follows them
    scores.copy_(to_device(inp2.scores, DEV))
    x.copy_(to_device(inp2.x, DEV))
    y_ref2 = to_host(eager.forward(to_device(inp2.scores, DEV), to_device(inp2.x, DEV), wgu, wd, **sc))
    torch.cuda.synchronize()
    for rep in range(2):
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), y_ref2), f"replay {rep} on new inputs"
    assert not np.array_equal(y_ref, y_ref2)
