"""CPU oracle of EPLB placement and of the logical -> physical replica choice.

TEST INFRASTRUCTURE ONLY, like moe_oracle: the plain reference that the
library's native planner and its GPU remap kernel are checked against. Only
the test suite and the benchmark's CPU leg may use it; it shares no code with
the library.

Source: page "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠"
(anrans.github.io, ai-infra-handbooks serving/moe/ep-deploy), section
"EPLB 与路由约束". It describes two strategies built from the same three
steps:
  hierarchical -- (1) pack the expert groups onto the nodes, balanced by
  load, the same number of groups per node; (2) inside each node replicate
  the hottest experts (redundant experts); (3) pack each node's physical
  experts onto its GPUs, balanced, the same number per GPU. A group never
  spans nodes.
  global -- the same without nodes: replicate over all experts, pack onto
  all GPUs.
The packing takes items from heaviest to lightest and puts each into the
lightest pack that still has room; replication repeatedly adds a replica to
the expert whose load per replica is highest. Its simulation reports the
busiest GPU's load over the mean (a replicated expert's load split evenly
over its replicas) and the mean number of nodes a token is sent to, where a
token slot uses a replica on a node the token already goes to when there is
one, else the replica on the lowest-numbered node.

Readings where the page leaves a step open (ties): equal weights are taken
in increasing index order, equal pack totals go to the lower pack, equal
loads per replica to the expert listed first; floating point sums are
float64, accumulated in placement order. The functions below restate the
page's description (a selection of the heaviest item, heaps of open packs
and of loads per replica), not its listing.
"""
from __future__ import annotations

import heapq

import numpy as np

__all__ = ["balanced_pack", "replicate", "place", "gpu_loads", "remap", "nodes_per_token"]


def _heaviest_first(weights: list[float]) -> list[int]:
    """Item indices from heaviest to lightest, found by repeatedly taking the heaviest item
    not yet taken (equal weights: the lower index first)."""
    left = list(range(len(weights)))
    order = []
    while left:
        best = left[0]
        for i in left[1:]:
            if weights[i] > weights[best]:
                best = i
        order.append(best)
        left.remove(best)
    return order


def balanced_pack(weights, n_packs: int) -> list[list[int]]:
    """Indices of the items in each pack, in the order they were placed.

    Every pack receives len(weights) // n_packs items (len(weights) must be a
    multiple of n_packs). Items go heaviest first (equal weights: lower index
    first), each to the lightest pack that still has room (equal totals: the
    lower pack). The packs with room are kept in a heap keyed by (total, pack
    index); a pack leaves the heap when it is full.
    """
    w = [float(v) for v in weights]
    n = len(w)
    assert n % n_packs == 0
    room = n // n_packs
    packs: list[list[int]] = [[] for _ in range(n_packs)]
    open_packs = [(0.0, p) for p in range(n_packs)]
    heapq.heapify(open_packs)
    for item in _heaviest_first(w):
        total, p = heapq.heappop(open_packs)
        packs[p].append(item)
        if len(packs[p]) < room:
            heapq.heappush(open_packs, (total + w[item], p))
    return packs


def replicate(load, experts: list[int], n_physical: int) -> tuple[list[int], dict[int, int]]:
    """Replica counts for `experts` so that they fill n_physical slots.

    Starting from one replica each, a replica is added n_physical - len(experts)
    times to the expert with the highest load per replica (equal: the one that
    comes first in `experts`), taken from a heap keyed by (-load per replica,
    position in `experts`). Returns the physical list (each expert repeated by
    its count, in the order of `experts`) and the counts.
    """
    count = {e: 1 for e in experts}
    heap = [(-float(load[e]), pos) for pos, e in enumerate(experts)]
    heapq.heapify(heap)
    for _ in range(n_physical - len(experts)):
        _, pos = heapq.heappop(heap)
        e = experts[pos]
        count[e] += 1
        heapq.heappush(heap, (-(float(load[e]) / count[e]), pos))
    physical = [e for e in experts for _ in range(count[e])]
    return physical, count


def place(load, num_groups: int, num_nodes: int, num_gpus: int, num_physical: int,
          hierarchical: bool) -> list[list[int]]:
    """Logical expert of every physical slot, per GPU (GPU-major), by the page's strategy."""
    E = len(load)
    G = E // num_groups
    if hierarchical:
        group_load = []
        for g in range(num_groups):   # sequential float64 sum, expert order
            total = 0.0
            for e in range(g * G, (g + 1) * G):
                total += float(load[e])
            group_load.append(total)
        node_experts = [[e for g in groups for e in range(g * G, (g + 1) * G)]
                        for groups in balanced_pack(group_load, num_nodes)]
    else:
        node_experts = [list(range(E))]
    gpus: list[list[int]] = []
    for experts in node_experts:
        n_phys = num_physical * len(experts) // E
        n_gpus = num_gpus * len(experts) // E
        physical, count = replicate(load, experts, n_phys)
        weights = [float(load[e]) / count[e] for e in physical]
        for pack in balanced_pack(weights, n_gpus):
            gpus.append([physical[i] for i in pack])
    return gpus


def gpu_loads(load, gpus: list[list[int]]) -> np.ndarray:
    """Load of each GPU: each physical slot carries its expert's load over the expert's replica count."""
    count: dict[int, int] = {}
    for g in gpus:
        for e in g:
            count[e] = count.get(e, 0) + 1
    return np.array([sum(float(load[e]) / count[e] for e in g) for g in gpus], dtype=np.float64)


def remap(topk_ids, gpus: list[list[int]], num_nodes: int) -> np.ndarray:
    """Physical slot (GPU-major: gpu * slots_per_gpu + position) for every (token, slot).

    Per token, slots in order: among the replicas of the slot's expert that sit
    on a node the token already goes to, the lowest slot; if there is none, the
    lowest slot on the lowest-numbered node holding a replica, and that node is
    added to the token's nodes. Written as plain loops.
    """
    per_gpu = len(gpus[0])
    gpus_per_node = len(gpus) // num_nodes
    replicas: dict[int, list[int]] = {}
    for gi, g in enumerate(gpus):
        for pos, e in enumerate(g):
            replicas.setdefault(e, []).append(gi * per_gpu + pos)
    ids = np.asarray(topk_ids, dtype=np.int64)
    out = np.empty(ids.shape, dtype=np.int64)
    for t in range(ids.shape[0]):
        nodes: set[int] = set()
        for j in range(ids.shape[1]):
            slots = sorted(replicas[int(ids[t, j])])
            on_used = [s for s in slots if (s // per_gpu) // gpus_per_node in nodes]
            if on_used:
                out[t, j] = on_used[0]
            else:
                lowest_node = min((s // per_gpu) // gpus_per_node for s in slots)
                out[t, j] = min(s for s in slots if (s // per_gpu) // gpus_per_node == lowest_node)
                nodes.add(lowest_node)
    return out.astype(np.int32)


def nodes_per_token(physical_ids, slots_per_gpu: int, gpus_per_node: int) -> np.ndarray:
    """Number of distinct nodes among each token's physical slots."""
    node = (np.asarray(physical_ids, dtype=np.int64) // slots_per_gpu) // gpus_per_node
    return np.array([len(set(row.tolist())) for row in node])
