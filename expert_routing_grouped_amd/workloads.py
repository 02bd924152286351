"""Seeded synthetic workloads for the MoE expert layer.

This module only draws inputs. It holds none of the layer's arithmetic (no
routing, no sorting, no GEMM): both the HIP path and the CPU oracle take
their inputs from here and from nowhere else.

Draw recipe (the order of draws is part of the definition):

* Grouped routing workloads follow the seeded simulation on the page
  "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠"
  (anrans.github.io, section "EPLB 与路由约束"): a generator
  ``numpy.random.default_rng(seed)``; first a per-expert bias
  ``b = normal(0, bias_std, E)`` (float64), then uniform scores
  ``U = random((T, E))`` (float64), and the router input is
  ``float32(U + 0.15 * b)``.
* Then the activations ``x = standard_normal((T, d), float32)``.
* Then, expert by expert in local order, the fused gate_up weight
  ``0.02 * standard_normal((2I, d), float32)`` (rows [0, I) gate, rows
  [I, 2I) up), and after all of them, expert by expert, the down weight
  ``0.02 * standard_normal((d, I), float32)``.
* The capacity workload (routing and capped dispatch only) draws its scores
  the same way, with the shape of the capacity-factor example in section 4.3
  of the ch15 page ("第十五章：多节点大模型推理", se7en.mintlify.app).
* The FP8 workload draws x and the weights as above; x is rounded to bf16
  (the layer quantises it), the weights are stored as OCP e4m3 codes with
  one float32 scale per 128 x 128 block (scale = amax / 448, nearest e4m3
  value, ties to the even code).
* bf16 workloads round x and the weights to bf16 (round to nearest even);
  the toy workload keeps float32 and draws its router logits with
  ``standard_normal((T, E), float32)`` before x.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    E: int                 # experts in the whole layer
    top_k: int             # experts per token
    num_groups: int        # expert groups (1 = no group stage)
    topk_groups: int       # groups kept per token
    score_mode: str        # "softmax" (router logits) or "raw" (scores used as given)
    renormalize: bool      # selected weights divided by their sum
    bias_std: float        # std of the per-expert bias b_e (raw mode)
    hidden: int            # d; 0 = routing and permutation only
    inter: int             # I (per-expert intermediate width)
    expert_begin: int      # first expert owned by this GPU
    num_local: int         # experts owned by this GPU
    dtype: str             # "f32" or "bf16" for x, weights and outputs
    seed: int = 0
    capacity_factor: str | None = None   # per-expert cap C = ceil(c T k / E), c as an exact decimal
    weight_format: str = "same"          # "fp8_e4m3_b128": x and expert weights as e4m3 with block scales
    layout: str = "grouped"              # "masked": fixed slots of C rows per local expert
    overflow: str = "drop"               # "reroute": over-capacity slots go to the next-best expert;
                                         # "defer": they wait for a later round (of `rounds`)
    rounds: int = 1

    @property
    def has_ffn(self) -> bool:
        return self.hidden > 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, with the prefill share taken two ways: the expert
# group that receives the most assignments (experts 32-63 at seed 0, the
# busiest card that sets the layer time) and the literal experts 0-31.
WORKLOADS = {
    "toy_fp32": Workload("toy_fp32", T=128, E=8, top_k=2, num_groups=1, topk_groups=1,
                         score_mode="softmax", renormalize=False, bias_std=0.0,
                         hidden=256, inter=512, expert_begin=0, num_local=8, dtype="f32"),
    "route_permute": Workload("route_permute", T=4096, E=256, top_k=8, num_groups=8, topk_groups=4,
                              score_mode="raw", renormalize=True, bias_std=1.0,
                              hidden=0, inter=0, expert_begin=0, num_local=256, dtype="f32"),
    "decode_ep": Workload("decode_ep", T=512, E=256, top_k=8, num_groups=8, topk_groups=4,
                          score_mode="raw", renormalize=True, bias_std=1.0,
                          hidden=7168, inter=2048, expert_begin=0, num_local=8, dtype="bf16"),
    "decode_tp": Workload("decode_tp", T=512, E=256, top_k=8, num_groups=8, topk_groups=4,
                          score_mode="raw", renormalize=True, bias_std=1.0,
                          hidden=7168, inter=64, expert_begin=0, num_local=256, dtype="bf16"),
    "prefill_straggler": Workload("prefill_straggler", T=8192, E=256, top_k=8, num_groups=8, topk_groups=4,
                                  score_mode="raw", renormalize=True, bias_std=2.0,
                                  hidden=7168, inter=2048, expert_begin=32, num_local=32, dtype="bf16"),
    "prefill_literal": Workload("prefill_literal", T=8192, E=256, top_k=8, num_groups=8, topk_groups=4,
                                score_mode="raw", renormalize=True, bias_std=2.0,
                                hidden=7168, inter=2048, expert_begin=0, num_local=32, dtype="bf16"),
    # decode_ep on FP8 operands: e4m3 weights with float32 128 x 128 block
    # scales; the layer quantises x and h per row and 128 features.
    "decode_ep_fp8": Workload("decode_ep_fp8", T=512, E=256, top_k=8, num_groups=8, topk_groups=4,
                              score_mode="raw", renormalize=True, bias_std=1.0,
                              hidden=7168, inter=2048, expert_begin=0, num_local=8, dtype="bf16",
                              weight_format="fp8_e4m3_b128"),
    # decode_ep on the masked layout (fixed slots of C = ceil(2 T k / E) = 32 rows per local
    # expert, the busiest expert's load at seed 0, so nothing is dropped): the layout of the
    # grouped GEMM that the INFRA page measures on its EP32 shape (8 experts per card).
    "decode_ep_masked": Workload("decode_ep_masked", T=512, E=256, top_k=8, num_groups=8, topk_groups=4,
                                 score_mode="raw", renormalize=True, bias_std=1.0,
                                 hidden=7168, inter=2048, expert_begin=0, num_local=8, dtype="bf16",
                                 capacity_factor="2", layout="masked"),
    # The capacity-factor example of ch15 section 4.3 (T = 5600 tokens, k = 16
    # of E = 896 experts, c = 1.2: C = 120), routing and capped dispatch only:
    # no groups, scores drawn as above (the page gives no score distribution)
    # with a bias std of 0.1, which puts the hottest expert at 3.5x the mean
    # load, within the 2.9-4.0 busiest/mean range of the EPLB page's simulation.
    "capacity_route": Workload("capacity_route", T=5600, E=896, top_k=16, num_groups=1, topk_groups=1,
                               score_mode="raw", renormalize=True, bias_std=0.1,
                               hidden=0, inter=0, expert_begin=0, num_local=896, dtype="f32",
                               capacity_factor="1.2"),
}
# The same example with the next-best expert overflow policy (routing with capacity).
WORKLOADS["capacity_reroute"] = WORKLOADS["capacity_route"].replace(name="capacity_reroute", overflow="reroute")
# ... and with the overflow deferred to a second round (dispatch into two rounds of C rows).
WORKLOADS["capacity_deferred"] = WORKLOADS["capacity_route"].replace(name="capacity_deferred", overflow="defer",
                                                                     rounds=2)
# decode_ep with C = ceil(T k / E) = 16 and the overflow deferred to a second round: the two
# grouped FFN calls together compute every row of the dropless layer (the busiest local expert
# has 32 rows at seed 0).
WORKLOADS["decode_ep_deferred"] = WORKLOADS["decode_ep"].replace(name="decode_ep_deferred", capacity_factor="1",
                                                                 overflow="defer", rounds=2)
# prefill_straggler on FP8 operands (decode_ep_fp8's format: e4m3 weights with 128 x 128 block
# scales, x quantised per row in the step): the prefill-sized FP8 call, whose experts of more
# than 64 rows take the tiled path.
WORKLOADS["prefill_straggler_fp8"] = WORKLOADS["prefill_straggler"].replace(name="prefill_straggler_fp8",
                                                                           weight_format="fp8_e4m3_b128")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite by construction, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


# OCP FP8 E4M3 (no infinities; S.1111.111 is NaN; largest finite 448):
# the value of every code 0x00 .. 0x7E (the positive half; the sign is bit 7).
def _e4m3_positive_values() -> np.ndarray:
    v = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        v[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


_E4M3 = _e4m3_positive_values()
FP8_BLOCK = 128


def quantize_e4m3_blocks(w: np.ndarray, block_rows: int = 1):
    """w [..., R, K] float32 -> (codes uint8 [..., R, K], scales float32 [..., R / block_rows, K / 128]).

    One scale per block of block_rows rows by 128 consecutive k: scale =
    amax / 448 (1 for an all-zero block); each value is divided by its scale
    and stored as the nearest e4m3 value, ties to the even code (all in
    float32). Input preparation only: the layer takes the codes and scales as
    given.
    """
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape[-2], w.shape[-1]
    assert K % FP8_BLOCK == 0 and R % block_rows == 0
    lead = w.shape[:-2]
    flat = w.reshape((-1, block_rows, K // FP8_BLOCK, FP8_BLOCK))
    code = np.empty(flat.shape, dtype=np.uint8)
    scale = np.empty((flat.shape[0], K // FP8_BLOCK), dtype=np.float32)
    step = max(1, (1 << 19) // (block_rows * K))   # row blocks per pass (temporaries of ~2 MB)
    for b0 in range(0, flat.shape[0], step):
        blk = flat[b0:b0 + step]
        q = np.abs(blk)
        amax = q.max(axis=(1, 3))
        sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        q /= sc[:, None, :, None]
        np.minimum(q, np.float32(448.0), out=q)
        # q >= 2^-6: keep 3 mantissa bits of the float32 pattern, rounded to
        # nearest even (a carry moves into the exponent), and rebias the
        # exponent from 127 to 7; below 2^-6 the code is rint(q * 2^9).
        u = q.view(np.uint32)
        normal = ((u + np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)) - np.uint32(120 << 3)
        sub = np.rint(q * np.float32(512.0)).astype(np.uint32)
        c = np.where(q >= np.float32(2.0 ** -6), normal, sub).astype(np.uint8)
        c |= ((blk.view(np.uint32) >> np.uint32(31)).astype(np.uint8) << np.uint8(7))
        code[b0:b0 + step] = c
        scale[b0:b0 + step] = sc
    scale = scale.reshape(lead + (R // block_rows, K // FP8_BLOCK))
    return code.reshape(w.shape), scale


@dataclass
class Inputs:
    workload: Workload
    scores: np.ndarray                 # [T, E] float32 (router logits or raw scores)
    x: np.ndarray | None = None        # [T, d] float32, or uint16 bf16 bits
    w_gate_up: np.ndarray | None = None  # [E_loc, 2I, d] float32 or uint16 bf16 bits
    w_down: np.ndarray | None = None     # [E_loc, d, I]  float32 or uint16 bf16 bits
    # fp8 format: codes (uint8, same shapes as above) and scales [E_loc, N / 128, K / 128] float32
    w_gate_up_scale: np.ndarray | None = None
    w_down_scale: np.ndarray | None = None


def _weights(rng: np.random.Generator, n: int, shape: tuple, bf16: bool, fp8: bool = False):
    if fp8:
        codes = np.empty((n,) + shape, dtype=np.uint8)
        scales = np.empty((n, shape[0] // FP8_BLOCK, shape[1] // FP8_BLOCK), dtype=np.float32)
        for e in range(n):
            w = rng.standard_normal(shape, dtype=np.float32)
            w *= np.float32(0.02)
            codes[e], scales[e] = quantize_e4m3_blocks(w, FP8_BLOCK)
        return codes, scales
    out = np.empty((n,) + shape, dtype=np.uint16 if bf16 else np.float32)
    for e in range(n):
        w = rng.standard_normal(shape, dtype=np.float32)
        w *= np.float32(0.02)
        out[e] = f32_to_bf16_bits(w) if bf16 else w
    return out


def generate(w: Workload, with_ffn: bool = True) -> Inputs:
    """Draw the seeded inputs of workload ``w`` (see the module docstring for the recipe)."""
    rng = np.random.default_rng(w.seed)
    if w.score_mode == "softmax":
        scores = rng.standard_normal((w.T, w.E), dtype=np.float32)
    else:
        b = rng.normal(0.0, w.bias_std, w.E)
        u = rng.random((w.T, w.E))
        scores = (u + 0.15 * b).astype(np.float32)
    inp = Inputs(w, np.ascontiguousarray(scores))
    if not (w.has_ffn and with_ffn):
        return inp
    bf16 = w.dtype == "bf16"
    x = rng.standard_normal((w.T, w.hidden), dtype=np.float32)
    inp.x = f32_to_bf16_bits(x) if bf16 else x
    if w.weight_format == "fp8_e4m3_b128":
        inp.w_gate_up, inp.w_gate_up_scale = _weights(rng, w.num_local, (2 * w.inter, w.hidden), bf16, True)
        inp.w_down, inp.w_down_scale = _weights(rng, w.num_local, (w.hidden, w.inter), bf16, True)
        return inp
    inp.w_gate_up = _weights(rng, w.num_local, (2 * w.inter, w.hidden), bf16)
    inp.w_down = _weights(rng, w.num_local, (w.hidden, w.inter), bf16)
    return inp


def page_simulation_scores(T: int = 20000, E: int = 256, seed: int = 0) -> np.ndarray:
    """The router input of the page's seeded routing simulation (T = 20000, E = 256), as float32."""
    return generate(Workload("page_sim", T=T, E=E, top_k=8, num_groups=8, topk_groups=4,
                             score_mode="raw", renormalize=True, bias_std=1.0, hidden=0,
                             inter=0, expert_begin=0, num_local=E, dtype="f32", seed=seed)).scores


def tie_stress_scores(T: int, E: int, seed: int = 1, levels: int = 16) -> np.ndarray:
    """Scores in [0, 1] quantised to multiples of 1/levels, so equal values are common (+0 and -0 both occur)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, levels + 1, size=(T, E)).astype(np.float32) / np.float32(levels)
    zero = q == 0
    neg = rng.random((T, E)) < 0.5
    q[zero & neg] = np.float32(-0.0)
    return q
