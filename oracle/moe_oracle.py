"""CPU oracle of the MoE expert layer: route -> dispatch -> expert FFN -> combine.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the HIP
path is checked against. Only the test suite, the package's smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does,
and it shares no code with the HIP kernels or their binding.

Everything is numpy. Floating point work is done in float64 from exactly
decoded inputs (float32 or bf16 bit patterns), with no intermediate rounding,
except where a float decides an integer: routing compares the float32 scores
and the float32 group scores, as the GPU does.

Sources (web pages; section names as printed on them):

* [EPLB] "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠"
  (anrans.github.io, ai-infra-handbooks, serving/moe/ep-deploy), section
  "EPLB 与路由约束": DeepSeek-V3 group-limited routing -- 256 experts in 8
  groups, group score = sum of the group's two highest scores, keep 4
  groups, then pick 8 experts inside them -- and its seeded simulation
  (contiguous groups, bias b ~ N(0, 1), scores U(0,1) + 0.15 b, per-expert
  load as a bincount of the routed table).
* [CH15] "第十五章：多节点大模型推理——并行部署、解码优化与 MoE 路由"
  (se7en.mintlify.app, ch15), section 3.4 "Expert Parallelism (EP)":
  gating picks top-k experts per token, dispatch sends each token to its
  experts, combine returns results to token order and merges them;
  section 4.1: gating picks *logical* experts; section 4.3: the imbalance
  metric max_e n_e / mean_e n_e, the capacity factor C = ceil(c T k / E)
  with its worked example (T = 5600, k = 16 of E = 896 experts, c = 1.2:
  mean 100, C = 120) and the table of overflow policies.
* [TRACE] "追踪一个 Token 在 MoE 推理中穿越 TP/CP/SP/EP/DP/PP 的路径"
  (attain.fans), hop 4 "分发到两个专家": the combined output is the
  router-weighted sum of the selected experts' outputs,
  y = p5 E5(x) + p27 E27(x).
* [L6] "Lecture 6 · 并行" (semidirectx.com, cs349d lecture06), section 2.2:
  the MLP is W_gate, W_up (split along d_ff) and W_down.
* [P2] "推理 INFRA 方法论（2）：分布式推理：TP、DP、EP、CP 与 PP"
  (johneyzheng.top): the gate and up projections are fused into one GEMM
  with N = 2 I.

Readings where the pages leave a step open (each is also listed in the
design notes of the repository):

1. The gated MLP's activation is SiLU, silu(z) = z / (1 + exp(-z)),
   h = silu(gate) * up (the pages name the three matrices but not the
   activation).
2. The fused weight is [gate; up] stacked along N: rows [0, I) are the
   gate, rows [I, 2I) the up projection.
3. Ties: the page does not say how equal scores are ordered; here ties go
   to the lower index (groups and experts), and -0 equals +0.
4. Group scores are float32 sums of the two largest float32 scores (a
   duplicated maximum counts twice); the page sums in float64 -- the two
   readings route the page's 20000 tokens identically.
5. "Plain softmax top-2" (toy workload): selection on the logits,
   weights are the softmax probabilities over all experts, not
   renormalised unless asked.
6. Within one expert, rows keep assignment order a = t * k + j (a stable
   counting sort); any order gives the same combined output.
7. On one GPU's share of experts, tokens with no local expert get a zero
   output row; y is this GPU's partial sum.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "route_softmax_topk", "route_grouped", "route",
    "route_reroute", "dispatch", "expert_capacity", "dispatch_capacity", "dispatch_masked",
    "dispatch_deferred", "remap_capacity", "gather_rows",
    "expert_ffn", "expert_ffn_masked",
    "expert_ffn_rows", "combine", "layer",
]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _decode(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def route_softmax_topk(logits: np.ndarray, top_k: int, renormalize: bool = False):
    """Plain top-k gating on router logits [CH15 section 4.1].

    Selection: descending logit, ties to the lower expert index (on the
    float32 logits; softmax is monotone so the set is the same as on the
    probabilities). Weights: softmax over all E experts in float64, taken
    at the selected experts; divided by their sum if ``renormalize``.
    Returns (topk_ids int32 [T, k], topk_weights float64 [T, k]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k out of range")
    # A stable sort of the negated values orders by descending value and
    # keeps lower indices first among equal values.
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    l64 = logits.astype(np.float64)
    ex = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def _best_remaining(values: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Per row, the index of the highest value among the allowed columns; among equal values
    the lowest index (np.argmax returns the first maximum). -0 and +0 compare equal."""
    masked = np.where(allowed, values, -np.inf)
    return np.argmax(masked, axis=1)


def route_grouped(scores: np.ndarray, top_k: int, num_groups: int, topk_groups: int,
                  renormalize: bool = True):
    """Group-limited top-k routing [EPLB, section "EPLB 与路由约束"].

    The page's statement, taken step by step:
    1. The E experts form ``num_groups`` contiguous groups of G = E / num_groups.
    2. A group's score is the sum of its two highest scores: the maximum, plus
       the maximum of the members left after one member holding the maximum is
       set aside (so a duplicated maximum counts twice); float32 sum.
    3. The token keeps ``topk_groups`` groups: the best group, then the best of
       the remaining ones, and so on (ties: lower group index).
    4. It then picks ``top_k`` experts among the members of its kept groups the
       same way, one at a time, best remaining first (ties: lower expert
       index); the output slots are in that order.
    5. Weights are the selected raw scores, divided by their sum when
       ``renormalize`` (float64).
    With ``num_groups == 1`` steps 2-3 are skipped (plain top-k on scores).
    Returns (topk_ids int32 [T, k], topk_weights float64 [T, k]).
    """
    s = np.asarray(scores, dtype=np.float32)
    T, E = s.shape
    if num_groups < 1 or E % num_groups:
        raise ValueError("E must be a multiple of num_groups")
    G = E // num_groups
    if not 1 <= topk_groups <= num_groups or not 1 <= top_k <= topk_groups * G:
        raise ValueError("top_k / topk_groups out of range")
    rows = np.arange(T)
    eligible = np.ones((T, E), dtype=bool)
    if num_groups > 1:
        if G < 2:
            raise ValueError("groups need at least two experts for a top-2 group score")
        group_score = np.empty((T, num_groups), dtype=np.float32)
        for g in range(num_groups):
            members = s[:, g * G:(g + 1) * G]
            first = np.argmax(members, axis=1)                      # one member holding the maximum
            top1 = members[rows, first]
            rest = np.ones(members.shape, dtype=bool)
            rest[rows, first] = False
            top2 = np.where(rest, members, -np.inf).max(axis=1).astype(np.float32)
            group_score[:, g] = top1 + top2                         # float32 + float32 -> float32
        kept = np.zeros((T, num_groups), dtype=bool)
        for _ in range(topk_groups):
            best = _best_remaining(group_score, ~kept)
            kept[rows, best] = True
        eligible = np.zeros((T, E), dtype=bool)
        for g in range(num_groups):
            eligible[:, g * G:(g + 1) * G] = kept[:, g:g + 1]
    ids = np.empty((T, top_k), dtype=np.int64)
    for j in range(top_k):
        best = _best_remaining(s, eligible)
        ids[:, j] = best
        eligible[rows, best] = False
    w = s[rows[:, None], ids].astype(np.float64)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def route(scores, top_k, num_groups, topk_groups, score_mode, renormalize):
    if score_mode == "softmax":
        if num_groups != 1:
            raise ValueError("softmax gating is used without groups")
        return route_softmax_topk(scores, top_k, renormalize)
    return route_grouped(scores, top_k, num_groups, topk_groups, renormalize)


def dispatch(topk_ids: np.ndarray, expert_begin: int, num_local: int):
    """Counting-sort permutation of assignments to this GPU's experts [CH15 section 3.4, dispatch].

    Assignment a = t * k + j (token t, slot j) is local when its expert lies
    in [expert_begin, expert_begin + num_local). Local assignments are
    ordered by (local expert, a).
    Returns (counts [E_loc], offsets [E_loc + 1], sorted_assign [M],
    assign_pos [T * k] with -1 for non-local assignments), all int32.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    local = (flat >= expert_begin) & (flat < expert_begin + num_local)
    a_local = np.nonzero(local)[0]
    e_local = flat[a_local] - expert_begin
    sorted_assign = a_local[np.argsort(e_local, kind="stable")]
    counts = np.bincount(e_local, minlength=num_local)
    offsets = np.zeros(num_local + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    assign_pos = np.full(flat.shape[0], -1, dtype=np.int64)
    assign_pos[sorted_assign] = np.arange(sorted_assign.shape[0])
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_assign.astype(np.int32), assign_pos.astype(np.int32))


def expert_capacity(num_tokens: int, top_k: int, num_experts: int, factor) -> int:
    """Per-expert capacity C = ceil(c * T * k / E) [CH15 section 4.3, "Capacity Factor"].

    factor is taken as an exact rational (a fractions.Fraction, an int, or a
    decimal string such as "1.2"), so that the ceiling is not moved by binary
    rounding: c = 1.2 with T = 5600, k = 16, E = 896 gives exactly 120.
    """
    c = Fraction(factor)
    return math.ceil(c * num_tokens * top_k / num_experts)


def dispatch_capacity(topk_ids: np.ndarray, expert_begin: int, num_local: int, capacity: int):
    """Dispatch with a per-expert capacity and the drop policy [CH15 section 4.3, capacity
    factor and the table of overflow policies: drop / residual path].

    Each local expert keeps its first `capacity` assignments in assignment order
    a = t * k + j (first come, first served); later ones are dropped: they get
    no row (assign_pos = -1) and contribute nothing to the combine.
    Returns (counts = rows kept per expert, offsets, sorted_assign [M],
    assign_pos [T * k], demand = assignments per expert before the cap), int32.
    Written as one pass over the assignments in order, with a running count
    per expert.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    demand = np.zeros(num_local, dtype=np.int64)
    kept = [[] for _ in range(num_local)]
    for a, expert in enumerate(flat.tolist()):
        e = expert - expert_begin
        if 0 <= e < num_local:
            if demand[e] < capacity:
                kept[e].append(a)
            demand[e] += 1
    counts = np.array([len(r) for r in kept], dtype=np.int64)
    offsets = np.zeros(num_local + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    sorted_assign = np.array([a for r in kept for a in r], dtype=np.int64)
    assign_pos = np.full(flat.shape[0], -1, dtype=np.int64)
    assign_pos[sorted_assign] = np.arange(sorted_assign.shape[0])
    return (counts.astype(np.int32), offsets.astype(np.int32), sorted_assign.astype(np.int32),
            assign_pos.astype(np.int32), demand.astype(np.int32))


def dispatch_deferred(topk_ids: np.ndarray, expert_begin: int, num_local: int, capacity: int,
                      rounds: int):
    """Dispatch with a per-expert capacity and the "defer to a second round" overflow policy
    [CH15 section 4.3, table of overflow policies: the assignment keeps its expert and is
    processed later].

    The assignments of local expert e, in assignment order a = t * k + j, fill round 0 up to
    `capacity`, then round 1, and so on: the i-th of them (from 0) goes to round i // C. Ones
    past `rounds` rounds are dropped (no row, assign_pos = -1); with C = 0 all are. Rows are
    laid out round after round, and inside a round expert after expert, each expert's rows in
    assignment order. Returns (round_counts [rounds, num_local], round_offsets [rounds,
    num_local + 1] (absolute rows: round r starts where round r - 1 ends), sorted_assign [M],
    assign_pos [T * k], demand [num_local] = assignments per expert), int32.
    Written as one pass over the assignments with a running count per expert.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    demand = [0] * num_local
    rows = [[[] for _ in range(num_local)] for _ in range(rounds)]
    for a, expert in enumerate(flat.tolist()):
        e = expert - expert_begin
        if 0 <= e < num_local:
            r = demand[e] // capacity if capacity > 0 else rounds
            if r < rounds:
                rows[r][e].append(a)
            demand[e] += 1
    counts = np.zeros((rounds, num_local), dtype=np.int64)
    offsets = np.zeros((rounds, num_local + 1), dtype=np.int64)
    order = []
    row = 0
    for r in range(rounds):
        for e in range(num_local):
            offsets[r, e] = row
            counts[r, e] = len(rows[r][e])
            order.extend(rows[r][e])
            row += len(rows[r][e])
        offsets[r, num_local] = row
    sorted_assign = np.array(order, dtype=np.int64)
    assign_pos = np.full(flat.shape[0], -1, dtype=np.int64)
    assign_pos[sorted_assign] = np.arange(sorted_assign.shape[0])
    return (counts.astype(np.int32), offsets.astype(np.int32), sorted_assign.astype(np.int32),
            assign_pos.astype(np.int32), np.array(demand, dtype=np.int32))


def remap_capacity(topk_ids: np.ndarray, replica_offsets: np.ndarray, replica_slots: np.ndarray,
                   capacity: int) -> np.ndarray:
    """Logical to physical expert with a per-replica capacity and the "send to a same-weight
    replica" overflow policy [CH15 section 4.3, table of overflow policies; section 4.4: the
    gating picks the logical expert, the system maps it to one of its identical replicas].

    Logical expert e's replicas are replica_slots[replica_offsets[e] : replica_offsets[e + 1]],
    in that order, each with room for `capacity` assignments. The assignments of e, in
    assignment order a = t * k + j, fill its first replica, then the next one: the i-th (from 0)
    goes to replica i // C. Past the room of all its replicas, for ids outside [0, E) and for
    experts without a replica the result is -1 (dropped). Written as one pass over the
    assignments with a running count per logical expert. Returns phys [T, k] int32.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    off = np.asarray(replica_offsets, dtype=np.int64)
    slots = np.asarray(replica_slots, dtype=np.int64)
    E = off.shape[0] - 1
    seen = [0] * E
    out = np.full(ids.shape, -1, dtype=np.int64)
    flat_out = out.reshape(-1)
    for a, e in enumerate(ids.reshape(-1).tolist()):
        if not 0 <= e < E:
            continue
        rep = seen[e] // capacity if capacity > 0 else off[e + 1] - off[e]
        if rep < off[e + 1] - off[e]:
            flat_out[a] = slots[off[e] + rep]
        seen[e] += 1
    return out.astype(np.int32)


def dispatch_masked(topk_ids: np.ndarray, expert_begin: int, num_local: int, capacity: int):
    """Dispatch into fixed per-expert slots, the "masked" layout of the grouped GEMM that the
    INFRA page measures ("推理 INFRA 方法论（2）", H20 paragraph: DeepGEMM masked), with the
    capacity and drop policy of CH15 section 4.3.

    Local expert e owns slot rows [e * C, (e + 1) * C) of a [num_local * C] buffer; its first C
    assignments in assignment order a = t * k + j take rows e * C, e * C + 1, ...; later ones
    are dropped. Written as one pass over the assignments with a running count per expert.
    Returns (counts = rows used per expert, slot_assign [num_local * C] = assignment in each
    slot row or -1 where empty, assign_pos [T * k] = slot row or -1, demand), int32.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    demand = np.zeros(num_local, dtype=np.int64)
    slot_assign = np.full(num_local * capacity, -1, dtype=np.int64)
    assign_pos = np.full(flat.shape[0], -1, dtype=np.int64)
    for a, expert in enumerate(flat.tolist()):
        e = expert - expert_begin
        if 0 <= e < num_local:
            if demand[e] < capacity:
                row = e * capacity + int(demand[e])
                slot_assign[row] = a
                assign_pos[a] = row
            demand[e] += 1
    counts = np.minimum(demand, capacity)
    return (counts.astype(np.int32), slot_assign.astype(np.int32), assign_pos.astype(np.int32),
            demand.astype(np.int32))


def expert_ffn_masked(x_slots: np.ndarray, counts: np.ndarray, capacity: int, w_gate_up: np.ndarray,
                      w_down: np.ndarray) -> np.ndarray:
    """The expert FFN on the masked layout: for local expert e only its first counts[e] slot rows,
    [e * C, e * C + counts[e]), go through the expert (the rest of its slots are padding and have
    no output). Returns o [num_local * C, d] float64 with zero rows where there is no output."""
    counts = np.asarray(counts, dtype=np.int64)
    E_loc = counts.shape[0]
    I = w_gate_up.shape[1] // 2
    out = np.zeros((E_loc * capacity, w_gate_up.shape[2]), dtype=np.float64)
    for e in range(E_loc):
        m = int(min(max(counts[e], 0), capacity))
        if m == 0:
            continue
        lo = e * capacity
        out[lo:lo + m] = _one_expert(_decode(x_slots[lo:lo + m]), w_gate_up[e], w_down[e], I)
    return out


def route_reroute(scores: np.ndarray, top_k: int, num_groups: int, topk_groups: int, capacity: int,
                  renormalize: bool = True):
    """Group-limited routing with a per-expert capacity and the "next-best expert" overflow
    policy [CH15 section 4.3, table of overflow policies: 转给次高分专家; EPLB page for the
    routing itself].

    Readings (the page names the policy only):
    1. Every token is routed as ``route_grouped``; its spare candidates are the next experts of
       the same ranking (its kept groups, descending score, lower index first), ranks k, k+1, ...
    2. Capacity goes first to the original choices: in assignment order a = t * k + j, an expert
       keeps its first C original assignments; the others overflow.
    3. Then, in assignment order, the i-th overflowing slot of a token (in slot order) moves to
       the token's spare candidate of rank k + i, which takes it if it holds fewer than C
       assignments at that moment; otherwise (or when the token has no such candidate) the slot
       is dropped: expert id -1, weight 0.
    4. Weights are the scores of each slot's final expert, divided by the sum over the token's
       slots that were not dropped when ``renormalize``.
    Returns (topk_ids int32 [T, k], topk_weights float64 [T, k], load int64 [E] = assignments
    each expert ends with). Written as plain loops over the assignments.
    """
    s = np.asarray(scores, dtype=np.float32)
    T, E = s.shape
    G = E // num_groups
    n_ranked = min(2 * top_k, topk_groups * G)
    ranked, _ = route_grouped(s, n_ranked, num_groups, topk_groups, renormalize=False)
    ids = ranked[:, :top_k].astype(np.int64).copy()
    load = np.zeros(E, dtype=np.int64)
    overflow = []
    for t in range(T):
        for j in range(top_k):
            e = int(ids[t, j])
            if load[e] < capacity:
                load[e] += 1
            else:
                overflow.append((t, j))
    nth = {}
    for t, j in overflow:
        i = nth.get(t, 0)
        nth[t] = i + 1
        r = top_k + i
        if r < n_ranked and load[int(ranked[t, r])] < capacity:
            ids[t, j] = int(ranked[t, r])
            load[int(ranked[t, r])] += 1
        else:
            ids[t, j] = -1
    w = np.where(ids >= 0, s[np.arange(T)[:, None], np.maximum(ids, 0)].astype(np.float64), 0.0)
    if renormalize:
        tot = w.sum(axis=1, keepdims=True)
        w = np.divide(w, tot, out=np.zeros_like(w), where=tot > 0)
    return ids.astype(np.int32), w, load


def gather_rows(x: np.ndarray, sorted_assign: np.ndarray, top_k: int) -> np.ndarray:
    """Row i of the permuted activations is the row of token sorted_assign[i] // k (exact copy)."""
    return np.asarray(x)[np.asarray(sorted_assign, dtype=np.int64) // top_k]


def _silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x_sorted: np.ndarray, offsets: np.ndarray, w_gate_up: np.ndarray,
               w_down: np.ndarray) -> np.ndarray:
    """Grouped SwiGLU expert FFN over the permuted rows [L6 section 2.2; P2 fused gate_up].

    For each local expert e with rows [offsets[e], offsets[e+1]):
    g = X Wg^T, u = X Wu^T with [Wg; Wu] = w_gate_up[e] ([2I, d]),
    h = silu(g) * u, o = h Wd^T with Wd = w_down[e] ([d, I]).
    Experts without rows are skipped. float64 throughout; returns o [M, d].
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E_loc = offsets.shape[0] - 1
    I = w_gate_up.shape[1] // 2
    d = w_gate_up.shape[2]
    out = np.zeros((int(offsets[-1]), d), dtype=np.float64)
    for e in range(E_loc):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        out[lo:hi] = _one_expert(_decode(x_sorted[lo:hi]), w_gate_up[e], w_down[e], I)
    return out


def _one_expert(xr: np.ndarray, wgu: np.ndarray, wd: np.ndarray, I: int) -> np.ndarray:
    wgu = _decode(wgu)
    g = xr @ wgu[:I].T
    u = xr @ wgu[I:].T
    h = _silu(g) * u
    return h @ _decode(wd).T


def expert_ffn_rows(x_rows: np.ndarray, local_expert: np.ndarray, w_gate_up: np.ndarray,
                    w_down: np.ndarray) -> np.ndarray:
    """The same FFN for an arbitrary set of rows: row r goes through local expert local_expert[r].

    Used to check sampled rows of large workloads one by one.
    """
    local_expert = np.asarray(local_expert, dtype=np.int64)
    I = w_gate_up.shape[1] // 2
    out = np.zeros((local_expert.shape[0], w_gate_up.shape[2]), dtype=np.float64)
    for e in np.unique(local_expert):
        sel = np.nonzero(local_expert == e)[0]
        out[sel] = _one_expert(_decode(np.asarray(x_rows)[sel]), w_gate_up[e], w_down[e], I)
    return out


def combine(o_sorted: np.ndarray, assign_pos: np.ndarray, topk_weights: np.ndarray) -> np.ndarray:
    """Gate-weighted combine back to token order [TRACE hop 4; CH15 section 3.4, combine].

    y[t] = sum over slots j (in order) with a local expert of
    topk_weights[t, j] * o_sorted[assign_pos[t * k + j]]; tokens with no
    local slot get zeros. float64.
    """
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = w.shape
    o = _decode(o_sorted) if np.asarray(o_sorted).dtype == np.uint16 else np.asarray(o_sorted, np.float64)
    pos = np.asarray(assign_pos, dtype=np.int64).reshape(T, k)
    y = np.zeros((T, o.shape[1] if o.ndim == 2 else 0), dtype=np.float64)
    for j in range(k):
        has = pos[:, j] >= 0
        y[has] += w[has, j, None] * o[pos[has, j]]
    return y


def layer(scores, x, w_gate_up, w_down, *, top_k, num_groups, topk_groups, score_mode,
          renormalize, expert_begin, num_local):
    """All four steps for one GPU's share; returns a dict of every intermediate."""
    ids, w = route(scores, top_k, num_groups, topk_groups, score_mode, renormalize)
    counts, offsets, sorted_assign, assign_pos = dispatch(ids, expert_begin, num_local)
    out = dict(topk_ids=ids, topk_weights=w, counts=counts, offsets=offsets,
               sorted_assign=sorted_assign, assign_pos=assign_pos)
    if x is not None:
        xs = gather_rows(x, sorted_assign, top_k)
        o = expert_ffn(xs, offsets, w_gate_up, w_down)
        out.update(x_sorted=xs, o_sorted=o, y=combine(o, assign_pos, w))
    return out
