"""CPU oracle of the FP8 variant of the expert layer: e4m3 codes with float32 block scales.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
the CPU-baseline leg of the benchmark may import it; the product path never
does, and it shares no code with the HIP kernels or their binding.

Sources:

* [EP] "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠"
  (anrans.github.io, ai-infra-handbooks, serving/moe/ep-deploy), section
  "双 batch 重叠": an expert's weights are counted as 44 MB of FP8 (one byte
  per weight for d = 7168, I = 2048), and a dispatched token is sent as FP8
  with its scales, 7168 + 224 bytes.
* [P2] "推理 INFRA 方法论（2）：分布式推理：TP、DP、EP、CP 与 PP"
  (johneyzheng.top): the measured fused gate_up grouped GEMM runs on FP8
  weights.
* [OFP8] The OCP 8-bit floating point specification, format E4M3: sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  subnormals m / 8 * 2^-6; S.1111.111 is NaN; there are no infinities, and
  the largest finite magnitude is 448 (S.1111.110).

Readings (each is also listed in the design notes of the repository):

1. Scale granularity: the pages give only the byte count of a token's
   scales, 224 B for 7168 features, which is one float32 per 128 features.
   Token rows (x, and the hidden activation h between the two GEMMs) take
   one scale per row and 128 consecutive features; weights take one per
   128 x 128 block (the pages count an expert's FP8 bytes as the weights
   alone). Dequantised value = decode(code) * scale.
2. Quantising a row block: scale = amax / 448 (float32; 1 when the block
   is all zero), code = the e4m3 value nearest to v / scale (float32
   division), ties to the even code, magnitudes above 448 saturate to 448;
   the sign bit is the sign bit of v. The decisions are taken in float32,
   the precision of the kernels.
3. h is quantised from float32 values: the GEMM's float64 result is
   rounded to float32 first (the kernels hold h in float32). Everything
   else is float64 from exactly decoded inputs.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "E4M3_MAX", "BLOCK", "e4m3_positive_values", "e4m3_decode", "e4m3_encode",
    "quantize_rows", "dequantize_rows", "dequantize_weights", "expert_ffn_fp8",
]

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_positive_values() -> np.ndarray:
    """Values of the codes 0 .. 126 (all finite non-negative codes), in code order [OFP8]."""
    out = np.empty(127, dtype=np.float64)
    for code in range(127):
        exp_field, mant = code >> 3, code & 7
        if exp_field == 0:
            out[code] = mant / 8.0 * 2.0 ** -6
        else:
            out[code] = (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return out


_POS = e4m3_positive_values()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values; the NaN codes (0x7F, 0xFF) decode to NaN [OFP8]."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = c & 0x7F
    val = np.where(mag == 0x7F, np.nan, _POS[np.minimum(mag, 126)])
    return np.where(c & 0x80, -val, val)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code to each finite float32 value, ties to the even code, saturating at 448.

    Chosen by comparing |v| with the two neighbouring entries of the value
    table (reading 2); the sign bit is copied from v.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v).astype(np.float64), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a (a <= 448 = _POS[126])
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - a
    d_lo = a - _POS[lo]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def quantize_rows(a: np.ndarray, block: int = BLOCK):
    """Rows [R, K] (float32 values) -> (codes uint8 [R, K], scales float32 [R, K / block]) (reading 2)."""
    a = np.asarray(a, dtype=np.float32)
    R, K = a.shape
    if K % block:
        raise ValueError("row length must be a multiple of the block")
    codes = np.empty((R, K), dtype=np.uint8)
    scales = np.empty((R, K // block), dtype=np.float32)
    for b in range(K // block):
        part = a[:, b * block:(b + 1) * block]
        amax = np.abs(part).max(axis=1)                                   # float32, exact
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = (part / s[:, None]).astype(np.float32)                        # float32 division
        codes[:, b * block:(b + 1) * block] = e4m3_encode(q)
        scales[:, b] = s
    return codes, scales


def dequantize_rows(codes: np.ndarray, scales: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Codes [R, K] and per-row block scales [R, K / block] -> float64 [R, K] (reading 1)."""
    vals = e4m3_decode(codes)
    return vals * np.repeat(np.asarray(scales, dtype=np.float64), block, axis=1)


def dequantize_weights(codes: np.ndarray, scales: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Codes [N, K] and block scales [N / block, K / block] -> float64 [N, K] (reading 1)."""
    s = np.asarray(scales, dtype=np.float64)
    full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)
    return e4m3_decode(codes) * full


def _silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn_fp8(x_codes, x_scales, row_index, row_div, offsets, w_gate_up, w_gate_up_scales,
                   w_down, w_down_scales, inter: int):
    """Grouped SwiGLU expert FFN on FP8 operands [EP section "双 batch 重叠"; P2; readings 1-3].

    Permuted row i is token row row_index[i] // row_div of (x_codes, x_scales)
    (row_index None: row i itself). For local expert e with rows
    [offsets[e], offsets[e+1]):
        X = dequant(x rows), W1 = dequant(w_gate_up[e]), W2 = dequant(w_down[e])
        [g | u] = X W1^T,  h = silu(g) * u               (float64)
        (hq, hs) = quantize_rows(float32(h))             (per row, 128 columns)
        o = dequant(hq, hs) W2^T                         (float64)
    Returns (o [M, hidden] float64, h_codes [M, I], h_scales [M, I / 128]).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    M = int(offsets[-1])
    rows = np.arange(M) if row_index is None else np.asarray(row_index, dtype=np.int64)[:M] // row_div
    xq = np.asarray(x_codes)[rows]
    xs = np.asarray(x_scales)[rows]
    hidden = xq.shape[1]
    o = np.zeros((M, hidden), dtype=np.float64)
    h_codes = np.zeros((M, inter), dtype=np.uint8)
    h_scales = np.ones((M, inter // BLOCK), dtype=np.float32)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = dequantize_rows(xq[lo:hi], xs[lo:hi])
        W1 = dequantize_weights(w_gate_up[e], w_gate_up_scales[e])
        g = X @ W1[:inter].T
        u = X @ W1[inter:].T
        h = _silu(g) * u
        hq, hs = quantize_rows(h.astype(np.float32))
        h_codes[lo:hi], h_scales[lo:hi] = hq, hs
        W2 = dequantize_weights(w_down[e], w_down_scales[e])
        o[lo:hi] = dequantize_rows(hq, hs) @ W2.T
    return o, h_codes, h_scales
