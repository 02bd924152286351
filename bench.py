"""Benchmark of one GPU's share of the MoE expert layer.

A step is one pass of the whole path over one batch of seeded synthetic input:
moe_route -> moe_dispatch (count, scan, permute, row gather) -> moe_expert_ffn
(gate_up GEMM + SiLU*up, down GEMM) -> moe_combine. The FP8 workload adds
moe_quantize_e4m3 of the token rows after the dispatch and runs
moe_expert_ffn_fp8 on e4m3 weights. Inputs are resident in HBM
before the timed region. Decode weight sets (0.35-0.7 GB) are comparable to
the 256 MB last-level cache, so the timed steps rotate over several copies of
the weights and every step reads its weights from HBM.

Prints one JSON line (rank 0, N = 1). The headline workload (decode_ep by
default) gives `value` and `roofline`; unless --headline-only is given the
same run also times the other graded shapes (prefill_straggler, MFMA-bound,
and decode_tp, HBM-bound), each with a roofline block of its own, under
`graded`. Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--headline-only] [--all]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from expert_routing_grouped_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
F32_PEAK_TFLOPS = 157.3      # MI355X fp32 vector, published
METRIC = "MoE layer tokens/s + grouped-GEMM %HBM-BW (decode) / %MFMA peak (prefill)"
HEADLINE = "decode_ep"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=HEADLINE, choices=sorted(W.WORKLOADS))
    p.add_argument("--all", action="store_true", help="also time every other workload")
    p.add_argument("--headline-only", action="store_true",
                   help="time only --workload (no graded prefill / decode_tp entries)")
    p.add_argument("--median-steps", type=int, default=100,
                   help="steps of the per-step pass whose median is reported beside the mean")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copies", type=int, default=0,
                   help="weight copies rotated over the timed steps (0 = enough to exceed the cache)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                   help="only run a plain device-to-device copy of MB megabytes, 5 times "
                        "(the known-size reference for hardware byte counters), and report its rate")
    p.add_argument("--operands", choices=["random", "zeros"], default="random",
                   help="zeros: a diagnostic run with x and the expert weights all zero (same routing), "
                        "which shows how much of the GEMM time depends on the operand values")
    return p.parse_args()


def calibrate_copy(mb, torch):
    n = mb * 1000 * 1000
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    ev[0].record(stream)
    for i in range(5):
        dst.copy_(src)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(5))
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 5, "median_us": us[2],
                      "read_plus_write_gbs": 2 * n / (us[2] * 1e-6) / 1e9}))


_CSRC = "expert_routing_grouped_amd/csrc/"
# Committed rocprofv3 counter records: workload -> (the sources of its FFN kernels, record file).
TRAFFIC_RECORDS = {
    "decode_ep": ([_CSRC + "ffn.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
                  os.path.join(ROOT, "profiles", "decode_ep_ffn_traffic.md")),
    "decode_tp": ([_CSRC + "ffn.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
                  os.path.join(ROOT, "profiles", "decode_tp_ffn_traffic.md")),
    "decode_ep_fp8": ([_CSRC + "ffn_fp8.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
                      os.path.join(ROOT, "profiles", "decode_ep_fp8_ffn_traffic.md")),
    "prefill_literal": ([_CSRC + "ffn.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
                        os.path.join(ROOT, "profiles", "prefill_literal_ffn_traffic.md")),
    "prefill_straggler": ([_CSRC + "ffn.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
                          os.path.join(ROOT, "profiles", "prefill_straggler_ffn_traffic.md")),
    "prefill_straggler_fp8": ([_CSRC + "ffn_fp8.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
                              os.path.join(ROOT, "profiles", "prefill_straggler_fp8_ffn_traffic.md")),
}


def measured_traffic(workload):
    """HBM bytes per FFN call from the committed rocprofv3 counter summary of this
    workload, or None when there is none or the kernel sources changed since."""
    import hashlib
    if workload not in TRAFFIC_RECORDS:
        return None
    sources, record = TRAFFIC_RECORDS[workload]
    try:
        rec = None
        for line in open(record):
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
        h = hashlib.sha256()
        for f in sources:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
    except (OSError, ValueError):
        return None
    if not rec or rec.get("workload") != workload or rec.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    return int(rec["traffic_bytes_per_call"])


def ffn_accounting(wl, counts):
    """Algorithmic FLOPs and HBM bytes of moe_expert_ffn for the measured routing."""
    counts = np.asarray(counts, dtype=np.int64)
    M = int(counts.sum())
    hit = int((counts > 0).sum())
    es = 2 if wl.dtype == "bf16" else 4
    d, I = wl.hidden, wl.inter
    flops = 6.0 * M * I * d
    weight_bytes = hit * 3.0 * I * d * es
    act_bytes = 2.0 * M * d * es            # permuted rows in, expert outputs out
    if wl.weight_format == "fp8_e4m3_b128":
        # e4m3 weights + one float32 scale per 128 x 128 block; FP8 rows with a
        # float32 scale per 128 features in, bf16 rows out
        weight_bytes = hit * 3.0 * I * d * (1 + 4 / 128 ** 2)
        act_bytes = M * d * (1 + 4 / 128) + M * d * 2.0
    return dict(M=M, hit=hit, flops=flops, bytes=weight_bytes + act_bytes,
                weight_bytes=weight_bytes, act_bytes=act_bytes)


def routing_stats(wl, topk_ids, counts):
    """Load statistics of the routed batch (ch15 page, section 4.3 "负载均衡"): the
    imbalance R = max_e n_e / mean_e n_e over all experts of the layer, and over
    this GPU's local experts; rows of the busiest local expert."""
    ids = np.asarray(topk_ids, dtype=np.int64).ravel()
    n_all = np.bincount(ids[ids >= 0], minlength=wl.E)      # dropped slots (-1) excluded
    counts = np.asarray(counts, dtype=np.int64)
    return dict(assignments=int(n_all.sum()), r_imbalance_all_experts=float(n_all.max() / n_all.mean()),
                r_imbalance_local=float(counts.max() / counts.mean()) if counts.sum() else 0.0,
                max_rows_per_local_expert=int(counts.max()))


def run_workload(wl, steps, warmup, copies, torch, moe, to_device, to_host, operands="random",
                 median_steps=100):
    dev = "cuda:0"
    t0 = time.time()
    inp = W.generate(wl)
    fp8 = wl.weight_format == "fp8_e4m3_b128"
    if operands == "zeros" and wl.has_ffn:   # same routing, all-zero GEMM operands
        inp.x = np.zeros_like(inp.x)
        inp.w_gate_up = np.zeros_like(inp.w_gate_up)
        inp.w_down = np.zeros_like(inp.w_down)
    gen_s = time.time() - t0
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    mode = moe.MOE_SCORE_SOFTMAX if wl.score_mode == "softmax" else moe.MOE_SCORE_RAW
    cap = None
    if wl.capacity_factor is not None:   # C = ceil(c T k / E), c an exact decimal
        from fractions import Fraction
        import math
        cap = math.ceil(Fraction(wl.capacity_factor) * wl.T * wl.top_k / wl.E)
    layer = moe.MoELayer(num_tokens=wl.T, num_experts=wl.E, top_k=wl.top_k,
                         num_groups=wl.num_groups, topk_groups=wl.topk_groups, score_mode=mode,
                         renormalize=wl.renormalize, expert_begin=wl.expert_begin,
                         num_local_experts=wl.num_local, hidden=wl.hidden, inter=wl.inter,
                         dtype=dt, device=dev,
                         expert_capacity=cap if (wl.layout != "masked" and wl.overflow == "drop") else None,
                         fp8=fp8, masked_capacity=cap if wl.layout == "masked" else None,
                         reroute_capacity=cap if wl.overflow == "reroute" else None,
                         deferred=(cap, wl.rounds) if wl.overflow == "defer" else None)
    scores = to_device(inp.scores, dev)
    x = to_device(inp.x, dev) if wl.has_ffn else None
    weights = []
    if wl.has_ffn:
        wbytes = (inp.w_gate_up.nbytes + inp.w_down.nbytes)
        n = copies or max(1, min(8, int(np.ceil(768e6 / wbytes)) + 1))
        for _ in range(n):
            if fp8:
                weights.append((to_device(inp.w_gate_up, dev), to_device(inp.w_down, dev),
                                to_device(inp.w_gate_up_scale, dev), to_device(inp.w_down_scale, dev)))
            else:
                weights.append((to_device(inp.w_gate_up, dev), to_device(inp.w_down, dev), None, None))
    else:
        weights.append((None, None, None, None))
    stream = torch.cuda.current_stream()

    def ffn(i):
        wgu, wd, wgs, wds = weights[i % len(weights)]
        layer.ffn(wgu, wd, x, w_gate_up_scales=wgs, w_down_scales=wds)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        layer.route(scores)
        if ev is not None:
            ev[1].record(stream)
        layer.dispatch(x)
        if fp8:
            layer.quantize(x)      # FP8 rows and scales, as the EP page dispatches them
        if ev is not None:
            ev[2].record(stream)
        if x is not None:
            ffn(i)
            if ev is not None:
                ev[3].record(stream)
            layer.combine()
        if ev is not None:
            ev[4].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # whole-step timing: no events inside
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / steps
    # per-call and per-step timing on the same stream (a separate pass of
    # n_med steps, events between the calls): medians
    n_med = max(steps, median_steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_med)]
    for i in range(n_med):
        step(i, evs[i])
    torch.cuda.synchronize()
    parts = np.zeros((n_med, 4))
    step_ms = np.zeros(n_med)
    for i, ev in enumerate(evs):
        parts[i] = [ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]),
                    ev[2].elapsed_time(ev[3]) if x is not None else 0.0,
                    ev[3].elapsed_time(ev[4]) if x is not None else 0.0]
        step_ms[i] = ev[0].elapsed_time(ev[4])
    parts_us = np.median(parts, axis=0) * 1e3
    ffn_us = None
    if x is not None:
        # moe_expert_ffn alone, back to back on the launch stream (the routing of
        # the last step stays in place): the per-launch duration of the roofline.
        # After the host-side pause above the chip's power management needs about
        # 15 calls of the prefill FFN (some 20 ms) to settle -- the first large-tile
        # calls after an idle gap run up to 45% slower -- so the calls are warmed up
        # for about 25 ms of GPU time (at least 2 calls) before they are timed.
        n_ffn = max(steps, 10)
        n_warm = int(min(max(2, 25e3 / max(parts_us[2], 1.0)), 2000))
        for i in range(n_warm):
            ffn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n_ffn):
            ffn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ffn_us = e0.elapsed_time(e1) / n_ffn * 1e3
    counts = to_host(layer.buf["counts"])
    round_counts = None
    if wl.overflow == "defer":   # rows per (round, expert); the FFN runs once per round
        round_counts = to_host(layer.buf["round_counts"])
        counts = round_counts.sum(0)
    res = dict(workload=wl.name, T=wl.T, ms_per_step=ms_per_step, wall_ms_per_step=wall / steps * 1e3,
               median_ms_per_step=float(np.median(step_ms)), median_over_steps=n_med,
               tokens_per_s=wl.T / (ms_per_step * 1e-3), gen_s=gen_s, weight_copies=len(weights),
               breakdown_us_median=dict(route=parts_us[0], dispatch=parts_us[1], ffn=parts_us[2],
                                        combine=parts_us[3]))
    res.update(routing_stats(wl, to_host(layer.buf["topk_ids"]), counts))
    res["assignments_per_s"] = res["assignments"] / (ms_per_step * 1e-3)
    res["local_rows_per_s"] = int(counts.sum()) / (ms_per_step * 1e-3)
    if wl.has_ffn:
        acc = ffn_accounting(wl, counts)
        if round_counts is not None:   # each round's call streams its hit experts' weights again
            per = [ffn_accounting(wl, rc) for rc in round_counts]
            acc = dict(acc, hit=sum(a["hit"] for a in per), bytes=sum(a["bytes"] for a in per),
                       weight_bytes=sum(a["weight_bytes"] for a in per))
        res["ffn_us_per_launch"] = ffn_us
        res["ffn_warmup_calls"] = n_warm
        t_ffn = ffn_us * 1e-6
        res.update(M=acc["M"], hit_experts=acc["hit"], ffn_gflop=acc["flops"] / 1e9,
                   ffn_bytes_mb=acc["bytes"] / 1e6,
                   ffn_tflops=acc["flops"] / t_ffn / 1e12, ffn_gbs=acc["bytes"] / t_ffn / 1e9,
                   layer_tflops=acc["flops"] / (ms_per_step * 1e-3) / 1e12)
        res["ffn_hbm_traffic_bytes"] = measured_traffic(wl.name)   # committed counter record, or None
        ai = acc["flops"] / acc["bytes"]
        res["mfma_peak_tflops"] = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
        res["ffn_bound"] = "mfma" if ai > res["mfma_peak_tflops"] * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
        if cap is not None:
            demand = to_host(layer.buf["demand"])
            res.update(capacity=cap, layout=wl.layout, dropped=int(demand.sum()) - acc["M"],
                       experts_over_capacity=int((demand > cap).sum()))
            if round_counts is not None:
                res.update(overflow="defer", rounds=wl.rounds, rows_per_round=round_counts.sum(1).tolist())
    else:
        M = int(counts.sum())
        route_bytes = wl.T * wl.E * 4 + wl.T * wl.top_k * 8
        res.update(M=M, route_gbs=route_bytes / (parts_us[0] * 1e-6) / 1e9)
        if cap is not None and wl.overflow == "reroute":
            ids = to_host(layer.buf["topk_ids"])
            res.update(capacity=cap, overflow="reroute", dropped=int((ids < 0).sum()),
                       max_load=int(to_host(layer.buf["expert_load"]).max()))
        elif cap is not None and round_counts is not None:
            demand = to_host(layer.buf["demand"])
            res.update(capacity=cap, overflow="defer", rounds=wl.rounds, assignments=int(demand.sum()),
                       rows_per_round=round_counts.sum(1).tolist(), dropped=int(demand.sum()) - M)
        elif cap is not None:
            demand = to_host(layer.buf["demand"])
            res.update(capacity=cap, assignments=int(demand.sum()), dropped=int(demand.sum()) - M,
                       experts_over_capacity=int((demand > cap).sum()))
    res["_inputs"] = inp
    return res


def run_eplb(torch, moe, to_device, to_host):
    """EPLB on the routed table of the EPLB page's simulation (20000 tokens, 256 experts in 8
    groups): the host planner for its two cluster shapes and strategies, and the GPU replica
    choice for all 20000 x 8 routed slots."""
    scores = torch.from_numpy(W.page_simulation_scores()).to("cuda:0")
    ids, _ = moe.moe_route(scores, 8, 8, 4)
    torch.cuda.synchronize()
    ids_h = to_host(ids)
    load = np.bincount(ids_h.ravel(), minlength=256).astype(float)
    out = {}
    stream = torch.cuda.current_stream()
    for nodes, gpus, phys in ((4, 32, 288), (8, 64, 320)):
        for hier in (False, True):
            t0 = time.perf_counter()
            p2l, offs, slots = moe.moe_eplb_place(load, 8, nodes, gpus, phys, hier)
            plan_us = (time.perf_counter() - t0) * 1e6
            d_offs, d_slots = to_device(offs, "cuda:0"), to_device(slots, "cuda:0")
            phys_ids = moe.moe_eplb_remap(ids, d_offs, d_slots, gpus, nodes)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                moe.moe_eplb_remap(ids, d_offs, d_slots, gpus, nodes, phys_ids)
            e1.record(stream)
            torch.cuda.synchronize()
            per = phys // gpus
            gpu_load = np.bincount(to_host(phys_ids).ravel() // per, minlength=gpus)
            # the same table with a per-replica capacity of 1.2 x the even share per slot and
            # the overflow sent on to the expert's next replica (ch15 section 4.3 table)
            C = int(-(-6 * ids_h.size // (5 * phys)))
            ws = torch.empty(moe.lib().moe_eplb_remap_capacity_workspace_size(ids.shape[0], 8, 256),
                             dtype=torch.uint8, device="cuda:0")
            cap_ids = moe.moe_eplb_remap_capacity(ids, d_offs, d_slots, C, workspace=ws)
            e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e2.record(stream)
            for _ in range(20):
                moe.moe_eplb_remap_capacity(ids, d_offs, d_slots, C, cap_ids, ws)
            e3.record(stream)
            torch.cuda.synchronize()
            cap_h = to_host(cap_ids).ravel()
            cap_load = np.bincount(cap_h[cap_h >= 0] // per, minlength=gpus)
            out[f"{nodes}n_{gpus}g_{'hier' if hier else 'global'}"] = dict(
                plan_us=plan_us, remap_us=e0.elapsed_time(e1) / 20 * 1e3,
                busiest_gpu_over_mean_after_remap=float(gpu_load.max() / gpu_load.mean()),
                replica_capacity=C, remap_capacity_us=e2.elapsed_time(e3) / 20 * 1e3,
                dropped_with_capacity=int((cap_h < 0).sum()),
                busiest_gpu_over_mean_with_capacity=float(cap_load.max() / cap_load.mean()))
    return out


def cpu_baseline(inp, wl, min_seconds=10.0):
    """The oracle as it stands, on the host cores: whole-layer passes over the
    workload, each step (route, dispatch, gather + expert FFN, combine) timed on
    its own, repeated until about min_seconds of CPU work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    fp8 = wl.weight_format == "fp8_e4m3_b128"
    if fp8:
        from oracle import fp8 as F
    step_s = dict(route=0.0, dispatch=0.0, ffn=0.0, combine=0.0)
    runs, t = 0, 0.0
    while runs == 0 or t < min_seconds:
        t0 = time.perf_counter()
        ids, w = oracle.route(inp.scores, wl.top_k, wl.num_groups, wl.topk_groups, wl.score_mode,
                              wl.renormalize)
        t1 = time.perf_counter()
        _, offsets, sa, pos = oracle.dispatch(ids, wl.expert_begin, wl.num_local)
        t2 = time.perf_counter()
        if fp8:
            xq, xs = F.quantize_rows(oracle.bf16_bits_to_f64(inp.x).astype(np.float32))
            o, _, _ = F.expert_ffn_fp8(xq, xs, sa, wl.top_k, offsets, inp.w_gate_up, inp.w_gate_up_scale,
                                       inp.w_down, inp.w_down_scale, wl.inter)
        else:
            o = oracle.expert_ffn(oracle.gather_rows(inp.x, sa, wl.top_k), offsets, inp.w_gate_up,
                                  inp.w_down)
        t3 = time.perf_counter()
        oracle.combine(o, pos, w)
        t4 = time.perf_counter()
        for name, dt in zip(step_s, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
            step_s[name] += dt
        t += t4 - t0
        runs += 1
    return {"value": wl.T * runs / t, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"{runs} passes of the whole {wl.name} layer ({wl.T} tokens each) through the "
                      f"numpy float64 oracle, {t:.1f} s; routing, dispatch and combine run on one "
                      f"thread, the expert FFN's matrix products on {blas} BLAS threads",
            "seconds": t, "host_cpus": os.cpu_count(),
            "host_cpus_usable": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "ms_per_pass_by_step": {k: v / runs * 1e3 for k, v in step_s.items()}}


def roofline_block(res, fp8):
    """Roofline of the dominant step (one moe_expert_ffn call) of a measured workload."""
    bound = res["ffn_bound"]
    if bound == "hbm":
        ach, peak, unit = res["ffn_gbs"], HBM_PEAK_GBS, "GB/s"
    else:
        ach, peak, unit = res["ffn_tflops"], res["mfma_peak_tflops"], "TFLOP/s"
    return {"bound": bound, "achieved": ach, "peak": peak, "unit": unit,
            "frac": ach / peak, "traffic": measured_traffic(res["workload"]),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": ("moe_expert_ffn_fp8 (gate_up GEMM + SiLU*up, h quantiser, down GEMM)"
                       if fp8 else "moe_expert_ffn (gate_up GEMM + SiLU*up, down GEMM)"),
            "us_per_launch": res["ffn_us_per_launch"],
            "algorithmic_bytes": res["ffn_bytes_mb"] * 1e6,
            "algorithmic_flops": res["ffn_gflop"] * 1e9}


# The shapes whose FFN fractions are reported beside the headline decode_ep:
# prefill (MFMA-bound), the TP-sliced decode (HBM-bound) and prefill on FP8
# operands (MFMA-bound against the fp8 peak).
GRADED = ("prefill_straggler", "decode_tp", "prefill_straggler_fp8")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer; run it with --gpus 1 "
              "(no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    from expert_routing_grouped_amd import moe
    from expert_routing_grouped_amd.tensors import to_device, to_host
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, torch)
        return
    moe.lib()

    wl = W.WORKLOADS[args.workload]
    fp8 = wl.weight_format == "fp8_e4m3_b128"
    print(f"bench: workload {wl.name}, steps {args.steps}, warmup {args.warmup}", file=sys.stderr,
          flush=True)
    head = run_workload(wl, args.steps, args.warmup, args.copies, torch, moe, to_device, to_host,
                        args.operands, args.median_steps)
    inp = head.pop("_inputs")
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else ("bf16" if wl.dtype == "bf16" else "f32"),
        "data": "synthetic" if args.operands == "random" else "synthetic, all-zero GEMM operands (diagnostic)",
        "config": {"workload": wl.name, "tokens": wl.T, "experts": wl.E, "top_k": wl.top_k,
                   "groups": f"{wl.num_groups} keep {wl.topk_groups}", "hidden": wl.hidden,
                   "inter": wl.inter, "local_experts": f"[{wl.expert_begin}, {wl.expert_begin + wl.num_local})",
                   "parallelism": "one GPU's expert share"},
    }
    if wl.has_ffn:
        out["roofline"] = roofline_block(head, fp8)
    out["detail"] = {k: v for k, v in head.items() if k not in ("tokens_per_s",)}
    print(f"bench: {wl.name} {head['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline and wl.has_ffn and args.operands == "random":
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, wl)
    del inp
    if not args.headline_only:
        graded = {}
        for name in GRADED:
            if name == wl.name:
                continue
            print(f"bench: graded workload {name}", file=sys.stderr, flush=True)
            g = W.WORKLOADS[name]
            r = run_workload(g, args.steps, args.warmup, args.copies, torch, moe, to_device, to_host,
                             args.operands, args.median_steps)
            r.pop("_inputs")
            g_fp8 = g.weight_format == "fp8_e4m3_b128"
            entry = {"workload": name, "tokens": g.T, "local_experts": f"[{g.expert_begin}, "
                     f"{g.expert_begin + g.num_local})", "inter": g.inter,
                     "dtype": "fp8_e4m3" if g_fp8 else "bf16",
                     "ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"],
                     "roofline": roofline_block(r, g_fp8),
                     "detail": {k: v for k, v in r.items() if k not in ("tokens_per_s", "ms_per_step")}}
            graded[name] = entry
            print(f"bench: {name} {r['ms_per_step'] * 1e3:.1f} us/step, FFN {r['ffn_us_per_launch']:.1f} us "
                  f"({entry['roofline']['frac']:.3f} of {entry['roofline']['bound']} peak)",
                  file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        out["graded"] = graded
    if args.all:
        others = {}
        for name in W.WORKLOADS:
            if name == wl.name or (name in GRADED and not args.headline_only):
                continue
            print(f"bench: workload {name}", file=sys.stderr, flush=True)
            r = run_workload(W.WORKLOADS[name], max(5, args.steps // 2), max(2, args.warmup // 2),
                             args.copies, torch, moe, to_device, to_host)
            r.pop("_inputs")
            others[name] = r
            torch.cuda.empty_cache()
        print("bench: eplb", file=sys.stderr, flush=True)
        others["eplb"] = run_eplb(torch, moe, to_device, to_host)
        out["workloads"] = others
    print(json.dumps(out, default=float))


if __name__ == "__main__":
    main()
