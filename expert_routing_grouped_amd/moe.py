"""Python binding of libmoe_mi355x.so (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch supplies device memory and the current stream; the functions
allocate missing outputs with torch and pass raw device pointers.

There is no fallback: if the library is not built, or a call returns an
error status, a MoeError is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_RAW = 0, 1

# Every symbol include/moe.h declares: (name, restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGNATURES = {
    "moe_abi_version": (ctypes.c_int32, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route": (ctypes.c_int, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_route_reroute_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "moe_route_reroute": (ctypes.c_int, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_dispatch_workspace_size": (ctypes.c_size_t, [_I, _I, _I]),
    "moe_dispatch": (ctypes.c_int, [_P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "moe_dispatch_capacity": (ctypes.c_int, [_P, _I, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P,
                                             _P, _P, ctypes.c_size_t, _P]),
    "moe_dispatch_masked": (ctypes.c_int, [_P, _I, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]),
    "moe_expert_capacity": (ctypes.c_int, [_I, _I, _I, ctypes.c_int64, ctypes.c_int64, _P]),
    "moe_expert_ffn_masked_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "moe_expert_ffn_masked": (ctypes.c_int, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "moe_expert_ffn": (ctypes.c_int, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P,
                                      ctypes.c_size_t, _P]),
    "moe_expert_ffn_noalloc": (ctypes.c_int, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_quantize_e4m3": (ctypes.c_int, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_expert_ffn_fp8_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "moe_expert_ffn_fp8": (ctypes.c_int, [_P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P,
                                          ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_eplb_place": (ctypes.c_int, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_eplb_remap": (ctypes.c_int, [_P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_dispatch_deferred_workspace_size": (ctypes.c_size_t, [_I, _I, _I]),
    "moe_dispatch_deferred": (ctypes.c_int, [_P, _I, _I, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P,
                                             _P, ctypes.c_size_t, _P]),
    "moe_eplb_remap_capacity_workspace_size": (ctypes.c_size_t, [_I, _I, _I]),
    "moe_eplb_remap_capacity": (ctypes.c_int, [_P, _I, _I, _P, _P, _I, _I, _P, _P, ctypes.c_size_t, _P]),
}

_lib = None


class MoeError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises MoeError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m expert_routing_grouped_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(code: int) -> str:
    return lib().moe_status_string(code).decode()


def _check(code: int, name: str) -> None:
    if code != 0:
        raise MoeError(f"{name} failed: {status_string(code)} (status {code})")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    return t


def _at_least(t: torch.Tensor, n: int, name: str) -> torch.Tensor:
    """The kernels write or read n elements of t: refuse a smaller buffer."""
    if t.numel() < n:
        raise MoeError(f"{name} holds {t.numel()} elements, {n} needed")
    return t


def _shape(t: torch.Tensor, shape: tuple, name: str) -> torch.Tensor:
    if tuple(t.shape) != tuple(shape):
        raise MoeError(f"{name} has shape {tuple(t.shape)}, {tuple(shape)} needed")
    return t


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return MOE_BF16
    if dtype == torch.float32:
        return MOE_F32
    raise MoeError(f"unsupported dtype {dtype}")


def moe_route(scores, top_k, num_groups=1, topk_groups=1, score_mode=MOE_SCORE_RAW,
              renormalize=True, topk_ids=None, topk_weights=None, stream=None):
    """topk_ids [T, k] int32, topk_weights [T, k] float32 (see moe_route in include/moe.h)."""
    _dev(scores, torch.float32, "scores")
    T, E = scores.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=scores.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, top_k), dtype=torch.float32, device=scores.device)
    _shape(_dev(topk_ids, torch.int32, "topk_ids"), (T, top_k), "topk_ids")
    _shape(_dev(topk_weights, torch.float32, "topk_weights"), (T, top_k), "topk_weights")
    _check(lib().moe_route(_ptr(scores), T, E, top_k, num_groups, topk_groups, score_mode,
                           int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_weights),
                           _stream(stream)), "moe_route")
    return topk_ids, topk_weights


def moe_route_reroute(scores, top_k, capacity, num_groups=1, topk_groups=1, renormalize=True,
                      topk_ids=None, topk_weights=None, expert_load=None, workspace=None, stream=None):
    """Routing with a per-expert capacity and the next-best expert overflow policy (RAW scores).
    Returns (topk_ids [T, k] int32 with -1 for dropped slots, topk_weights [T, k], expert_load [E])."""
    _dev(scores, torch.float32, "scores")
    T, E = scores.shape
    dev = scores.device
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    if expert_load is None:
        expert_load = torch.empty(E, dtype=torch.int32, device=dev)
    _shape(_dev(topk_ids, torch.int32, "topk_ids"), (T, top_k), "topk_ids")
    _shape(_dev(topk_weights, torch.float32, "topk_weights"), (T, top_k), "topk_weights")
    _at_least(_dev(expert_load, torch.int32, "expert_load"), E, "expert_load")
    need = int(lib().moe_route_reroute_workspace_size(T, E, top_k, num_groups, topk_groups))
    if T and need == 0:
        raise MoeError("moe_route_reroute: unsupported sizes")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().moe_route_reroute(_ptr(scores), T, E, top_k, num_groups, topk_groups, int(bool(renormalize)),
                                   int(capacity), _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_load),
                                   _ptr(workspace), workspace.numel(), _stream(stream)), "moe_route_reroute")
    return topk_ids, topk_weights, expert_load


def moe_dispatch(topk_ids, expert_begin, num_local_experts, x=None, out=None, stream=None,
                 capacity=None):
    """Counting-sort dispatch. Returns dict(counts, offsets, sorted_assign, assign_pos, x_sorted).

    With capacity = C (an int) it calls moe_dispatch_capacity: each expert keeps its first C
    assignments, counts are clamped and the result also holds demand (assignments per expert
    before the cap)."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    o = dict(out or {})
    n = T * k
    o.setdefault("counts", torch.empty(num_local_experts, dtype=torch.int32, device=dev))
    o.setdefault("offsets", torch.empty(num_local_experts + 1, dtype=torch.int32, device=dev))
    o.setdefault("sorted_assign", torch.empty(max(n, 1), dtype=torch.int32, device=dev))
    o.setdefault("assign_pos", torch.empty(max(n, 1), dtype=torch.int32, device=dev))
    hidden, dtype = 0, MOE_BF16
    if x is not None:
        dtype = _code(x.dtype)
        _dev(x, x.dtype, "x")
        if x.dim() != 2 or x.shape[0] < T:
            raise MoeError(f"x must be [>= {T}, hidden], got {tuple(x.shape)}")
        hidden = x.shape[1]
        o.setdefault("x_sorted", torch.empty((max(n, 1), hidden), dtype=x.dtype, device=dev))
        _dev(o["x_sorted"], x.dtype, "x_sorted")
        if o["x_sorted"].dim() != 2 or o["x_sorted"].shape[1] != hidden or o["x_sorted"].shape[0] < n:
            raise MoeError(f"x_sorted must be [>= {n}, {hidden}], got {tuple(o['x_sorted'].shape)}")
    else:
        o["x_sorted"] = None
    for name, need_n in (("counts", num_local_experts), ("offsets", num_local_experts + 1),
                         ("sorted_assign", n), ("assign_pos", n)):
        _at_least(_dev(o[name], torch.int32, name), need_n, name)
    need = int(lib().moe_dispatch_workspace_size(T, k, num_local_experts))
    ws = o.get("workspace")
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(ws if need else None)
    ws_bytes = ws.numel() if (need and ws is not None) else 0
    if capacity is None:
        _check(lib().moe_dispatch(_ptr(topk_ids), T, k, expert_begin, num_local_experts, _ptr(x),
                                  hidden, dtype, _ptr(o["counts"]), _ptr(o["offsets"]),
                                  _ptr(o["sorted_assign"]), _ptr(o["assign_pos"]),
                                  _ptr(o["x_sorted"]), ws_ptr, ws_bytes, _stream(stream)),
               "moe_dispatch")
        return o
    o.setdefault("demand", torch.empty(num_local_experts, dtype=torch.int32, device=dev))
    _at_least(_dev(o["demand"], torch.int32, "demand"), num_local_experts, "demand")
    _check(lib().moe_dispatch_capacity(_ptr(topk_ids), T, k, expert_begin, num_local_experts,
                                       int(capacity), _ptr(x), hidden, dtype, _ptr(o["counts"]),
                                       _ptr(o["offsets"]), _ptr(o["demand"]),
                                       _ptr(o["sorted_assign"]), _ptr(o["assign_pos"]),
                                       _ptr(o["x_sorted"]), ws_ptr, ws_bytes, _stream(stream)),
           "moe_dispatch_capacity")
    return o


def moe_dispatch_masked(topk_ids, expert_begin, num_local_experts, capacity, x=None, out=None,
                        stream=None):
    """Capped dispatch into fixed per-expert slots of `capacity` rows (the masked layout).

    Returns dict(counts, demand, slot_assign [E_loc * C], assign_pos [T * k], x_slots or None)."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    o = dict(out or {})
    n = T * k
    rows = num_local_experts * int(capacity)
    o.setdefault("counts", torch.empty(num_local_experts, dtype=torch.int32, device=dev))
    o.setdefault("demand", torch.empty(num_local_experts, dtype=torch.int32, device=dev))
    o.setdefault("slot_assign", torch.empty(max(rows, 1), dtype=torch.int32, device=dev))
    o.setdefault("assign_pos", torch.empty(max(n, 1), dtype=torch.int32, device=dev))
    for name, need_n in (("counts", num_local_experts), ("demand", num_local_experts),
                         ("slot_assign", rows), ("assign_pos", n)):
        _at_least(_dev(o[name], torch.int32, name), need_n, name)
    hidden, dtype = 0, MOE_BF16
    if x is not None:
        dtype = _code(x.dtype)
        _dev(x, x.dtype, "x")
        if x.dim() != 2 or x.shape[0] < T:
            raise MoeError(f"x must be [>= {T}, hidden], got {tuple(x.shape)}")
        hidden = x.shape[1]
        o.setdefault("x_slots", torch.empty((max(rows, 1), hidden), dtype=x.dtype, device=dev))
        xs = _dev(o["x_slots"], x.dtype, "x_slots")
        if xs.dim() != 2 or xs.shape[1] != hidden or xs.shape[0] < rows:
            raise MoeError(f"x_slots must be [>= {rows}, {hidden}], got {tuple(xs.shape)}")
    else:
        o["x_slots"] = None
    need = int(lib().moe_dispatch_workspace_size(T, k, num_local_experts))
    ws = o.get("workspace")
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().moe_dispatch_masked(_ptr(topk_ids), T, k, expert_begin, num_local_experts, int(capacity),
                                     _ptr(x), hidden, dtype, _ptr(o["counts"]), _ptr(o["demand"]),
                                     _ptr(o["slot_assign"]), _ptr(o["assign_pos"]), _ptr(o["x_slots"]),
                                     _ptr(ws if need else None), ws.numel() if need else 0, _stream(stream)),
           "moe_dispatch_masked")
    return o


def moe_expert_ffn_masked(x_slots, expert_counts, capacity, w_gate_up, w_down, o_slots=None,
                          workspace=None, stream=None):
    """Grouped SwiGLU FFN on the masked layout; returns o_slots [E_loc * C, d] (valid rows written)."""
    dt = x_slots.dtype
    _dev(x_slots, dt, "x_slots")
    _dev(expert_counts, torch.int32, "expert_counts")
    _dev(w_gate_up, dt, "w_gate_up")
    _dev(w_down, dt, "w_down")
    E_loc, two_i, d2 = w_gate_up.shape
    inter = two_i // 2
    hidden = x_slots.shape[1]
    rows = E_loc * int(capacity)
    _at_least(expert_counts, E_loc, "expert_counts")
    if d2 != hidden or tuple(w_down.shape) != (E_loc, hidden, inter):
        raise MoeError("weight shapes do not match x_slots")
    if x_slots.shape[0] < rows:
        raise MoeError(f"x_slots holds {x_slots.shape[0]} rows, {rows} needed")
    if o_slots is None:
        o_slots = torch.zeros((max(rows, 1), hidden), dtype=dt, device=x_slots.device)
    _dev(o_slots, dt, "o_slots")
    if o_slots.shape[0] < rows or o_slots.shape[1] != hidden:
        raise MoeError(f"o_slots must be [>= {rows}, {hidden}]")
    need = int(lib().moe_expert_ffn_masked_workspace_size(E_loc, hidden, inter, int(capacity), _code(dt)))
    if need == 0:
        raise MoeError("moe_expert_ffn_masked: unsupported sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_slots.device)
    _check(lib().moe_expert_ffn_masked(_ptr(x_slots), _ptr(expert_counts), int(capacity), _ptr(w_gate_up),
                                       _ptr(w_down), E_loc, hidden, inter, _code(dt), _ptr(o_slots),
                                       _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_expert_ffn_masked")
    return o_slots


def moe_expert_capacity(num_tokens, top_k, num_experts, factor_num, factor_den=1) -> int:
    """C = ceil(c T k / E) with c = factor_num / factor_den exactly (host only)."""
    out = ctypes.c_int32(0)
    _check(lib().moe_expert_capacity(int(num_tokens), int(top_k), int(num_experts), int(factor_num),
                                     int(factor_den), ctypes.byref(out)), "moe_expert_capacity")
    return int(out.value)


def ffn_workspace_size(num_local_experts, hidden, inter, row_capacity, dtype) -> int:
    code = _code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().moe_expert_ffn_workspace_size(num_local_experts, hidden, inter,
                                                   row_capacity, code))


def moe_expert_ffn(x, expert_offsets, w_gate_up, w_down, row_index=None, row_index_div=1,
                   row_capacity=None, o_sorted=None, workspace=None, stream=None):
    """Grouped SwiGLU FFN over the permuted rows; returns o_sorted [row_capacity, d].

    x is x_sorted (row_index None) or the token rows, read through row_index
    (sorted_assign) and row_index_div (top_k): the dispatch gather fused into the GEMM.
    """
    dt = x.dtype
    _dev(x, dt, "x")
    _dev(expert_offsets, torch.int32, "expert_offsets")
    _dev(w_gate_up, dt, "w_gate_up")
    _dev(w_down, dt, "w_down")
    if row_index is not None:
        _dev(row_index, torch.int32, "row_index")
        cap = row_index.numel() if row_capacity is None else row_capacity
        _at_least(row_index, cap, "row_index")
    else:
        cap = x.shape[0] if row_capacity is None else row_capacity
    hidden = x.shape[1]
    E_loc, two_i, d2 = w_gate_up.shape
    _at_least(expert_offsets, E_loc + 1, "expert_offsets")
    inter = two_i // 2
    if d2 != hidden or tuple(w_down.shape) != (E_loc, hidden, inter):
        raise MoeError("weight shapes do not match x")
    if o_sorted is None:
        o_sorted = torch.empty((max(cap, 1), hidden), dtype=dt, device=x.device)
    _dev(o_sorted, dt, "o_sorted")
    if o_sorted.shape[0] < cap or (row_index is None and x.shape[0] < cap):
        raise MoeError("row buffers are smaller than row_capacity")
    need = ffn_workspace_size(E_loc, hidden, inter, cap, dt)
    if need == 0:
        raise MoeError("moe_expert_ffn: unsupported sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib().moe_expert_ffn(_ptr(x), _ptr(row_index), int(row_index_div), _ptr(expert_offsets),
                                _ptr(w_gate_up), _ptr(w_down), E_loc, hidden, inter, cap, _code(dt),
                                _ptr(o_sorted), _ptr(workspace), workspace.numel(),
                                _stream(stream)), "moe_expert_ffn")
    return o_sorted


MOE_ERR_SCRATCH = 5
NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_expert_ffn_noalloc(x, expert_offsets, w_gate_up, w_down, o_sorted, row_index=None,
                           row_index_div=1, row_capacity=None, stream=None):
    """moe_expert_ffn with the library's fixed scratch instead of a workspace (no allocation:
    o_sorted must be supplied). Raises MoeError for sizes whose workspace exceeds the scratch."""
    dt = x.dtype
    _dev(x, dt, "x")
    _dev(expert_offsets, torch.int32, "expert_offsets")
    _dev(w_gate_up, dt, "w_gate_up")
    _dev(w_down, dt, "w_down")
    _dev(o_sorted, dt, "o_sorted")
    if row_index is not None:
        _dev(row_index, torch.int32, "row_index")
        cap = row_index.numel() if row_capacity is None else row_capacity
        _at_least(row_index, cap, "row_index")
    else:
        cap = x.shape[0] if row_capacity is None else row_capacity
    hidden = x.shape[1]
    E_loc, two_i, d2 = w_gate_up.shape
    inter = two_i // 2
    _at_least(expert_offsets, E_loc + 1, "expert_offsets")
    if d2 != hidden or tuple(w_down.shape) != (E_loc, hidden, inter):
        raise MoeError("weight shapes do not match x")
    if o_sorted.shape[0] < cap or o_sorted.shape[1] != hidden or (row_index is None and x.shape[0] < cap):
        raise MoeError("row buffers are smaller than row_capacity")
    _check(lib().moe_expert_ffn_noalloc(_ptr(x), _ptr(row_index), int(row_index_div), _ptr(expert_offsets),
                                        _ptr(w_gate_up), _ptr(w_down), E_loc, hidden, inter, cap, _code(dt),
                                        _ptr(o_sorted), _stream(stream)), "moe_expert_ffn_noalloc")
    return o_sorted


def moe_quantize_e4m3(x, codes=None, scales=None, stream=None):
    """Rows of x [R, C] (float32 or bf16) -> (e4m3 codes uint8 [R, C], scales float32 [R, C / 128])."""
    _dev(x, x.dtype, "x")
    R, C = x.shape
    if codes is None:
        codes = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((R, C // 128), dtype=torch.float32, device=x.device)
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.float32, "scales")
    if tuple(codes.shape) != (R, C) or scales.numel() < R * (C // 128):
        raise MoeError("moe_quantize_e4m3: output shapes do not match x")
    _check(lib().moe_quantize_e4m3(_ptr(x), R, C, _code(x.dtype), _ptr(codes), _ptr(scales),
                                   _stream(stream)), "moe_quantize_e4m3")
    return codes, scales


def ffn_fp8_workspace_size(num_local_experts, hidden, inter, row_capacity) -> int:
    return int(lib().moe_expert_ffn_fp8_workspace_size(num_local_experts, hidden, inter, row_capacity))


def moe_expert_ffn_fp8(x_codes, x_scales, expert_offsets, w_gate_up, w_gate_up_scales, w_down,
                       w_down_scales, row_index=None, row_index_div=1, row_capacity=None,
                       o_sorted=None, workspace=None, stream=None):
    """Grouped SwiGLU FFN on e4m3 operands with float32 block scales; returns o_sorted (bf16)."""
    _dev(x_codes, torch.uint8, "x_codes")
    _dev(x_scales, torch.float32, "x_scales")
    _dev(expert_offsets, torch.int32, "expert_offsets")
    _dev(w_gate_up, torch.uint8, "w_gate_up")
    _dev(w_down, torch.uint8, "w_down")
    _dev(w_gate_up_scales, torch.float32, "w_gate_up_scales")
    _dev(w_down_scales, torch.float32, "w_down_scales")
    if row_index is not None:
        _dev(row_index, torch.int32, "row_index")
        cap = row_index.numel() if row_capacity is None else row_capacity
        _at_least(row_index, cap, "row_index")
    else:
        cap = x_codes.shape[0] if row_capacity is None else row_capacity
    hidden = x_codes.shape[1]
    E_loc, two_i, d2 = w_gate_up.shape
    _at_least(expert_offsets, E_loc + 1, "expert_offsets")
    inter = two_i // 2
    if d2 != hidden or tuple(w_down.shape) != (E_loc, hidden, inter):
        raise MoeError("weight shapes do not match x")
    if tuple(w_gate_up_scales.shape) != (E_loc, two_i // 128, hidden // 128) or \
            tuple(w_down_scales.shape) != (E_loc, hidden // 128, inter // 128):
        raise MoeError("weight scale shapes do not match the weights")
    if tuple(x_scales.shape) != (x_codes.shape[0], hidden // 128):
        raise MoeError("x_scales shape does not match x_codes")
    if o_sorted is None:
        o_sorted = torch.empty((max(cap, 1), hidden), dtype=torch.bfloat16, device=x_codes.device)
    _dev(o_sorted, torch.bfloat16, "o_sorted")
    if o_sorted.shape[0] < cap or (row_index is None and x_codes.shape[0] < cap):
        raise MoeError("row buffers are smaller than row_capacity")
    need = ffn_fp8_workspace_size(E_loc, hidden, inter, cap)
    if need == 0:
        raise MoeError("moe_expert_ffn_fp8: unsupported sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_codes.device)
    _check(lib().moe_expert_ffn_fp8(_ptr(x_codes), _ptr(x_scales), _ptr(row_index), int(row_index_div),
                                    _ptr(expert_offsets), _ptr(w_gate_up), _ptr(w_gate_up_scales),
                                    _ptr(w_down), _ptr(w_down_scales), E_loc, hidden, inter, cap,
                                    _ptr(o_sorted), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "moe_expert_ffn_fp8")
    return o_sorted


def moe_combine(o_sorted, assign_pos, topk_weights, out_dtype=None, y=None, stream=None):
    """y [T, d] = router-weighted sum of each token's local expert outputs."""
    _dev(o_sorted, o_sorted.dtype, "o_sorted")
    _dev(assign_pos, torch.int32, "assign_pos")
    _dev(topk_weights, torch.float32, "topk_weights")
    T, k = topk_weights.shape
    hidden = o_sorted.shape[1]
    _at_least(assign_pos, T * k, "assign_pos")
    out_dtype = out_dtype or o_sorted.dtype
    if y is None:
        y = torch.empty((T, hidden), dtype=out_dtype, device=o_sorted.device)
    _shape(_dev(y, out_dtype, "y"), (T, hidden), "y")
    _check(lib().moe_combine(_ptr(o_sorted), _ptr(assign_pos), _ptr(topk_weights), T, k, hidden,
                             _code(o_sorted.dtype), _code(out_dtype), _ptr(y), _stream(stream)),
           "moe_combine")
    return y


def moe_eplb_place(load, num_groups, num_nodes, num_gpus, num_physical, hierarchical):
    """EPLB placement on the host (see moe_eplb_place in include/moe.h).

    load: per-expert loads (any array-like, converted to float64 on the host).
    Returns numpy int32 arrays (phys_to_logical [P], replica_offsets [E + 1], replica_slots [P]).
    """
    import numpy as np
    ld = np.ascontiguousarray(np.asarray(load, dtype=np.float64))
    E = ld.shape[0]
    p2l = np.empty(num_physical, dtype=np.int32)
    offs = np.empty(E + 1, dtype=np.int32)
    slots = np.empty(num_physical, dtype=np.int32)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(lib().moe_eplb_place(ptr(ld), E, num_groups, num_nodes, num_gpus, num_physical,
                                int(bool(hierarchical)), ptr(p2l), ptr(offs), ptr(slots)),
           "moe_eplb_place")
    return p2l, offs, slots


def moe_eplb_remap(topk_ids, replica_offsets, replica_slots, num_gpus, num_nodes, physical_ids=None,
                   stream=None):
    """Physical slot per routed (token, slot); the replica table given as device tensors."""
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(replica_offsets, torch.int32, "replica_offsets")
    _dev(replica_slots, torch.int32, "replica_slots")
    T, k = topk_ids.shape
    if physical_ids is None:
        physical_ids = torch.empty_like(topk_ids)
    _shape(_dev(physical_ids, torch.int32, "physical_ids"), (T, k), "physical_ids")
    if replica_offsets.numel() < 2 or replica_slots.numel() < 1:
        raise MoeError("the replica table is empty")
    _check(lib().moe_eplb_remap(_ptr(topk_ids), T, k, _ptr(replica_offsets), _ptr(replica_slots),
                                replica_offsets.numel() - 1, replica_slots.numel(), num_gpus,
                                num_nodes, _ptr(physical_ids), _stream(stream)), "moe_eplb_remap")
    return physical_ids


def moe_dispatch_deferred(topk_ids, expert_begin, num_local_experts, capacity, rounds, x=None, out=None,
                          stream=None):
    """Dispatch with the "defer to a later round" overflow policy: the i-th assignment of an
    expert goes to round i // capacity (dropped past `rounds` rounds). Returns dict(round_counts
    [rounds, E_loc], round_offsets [rounds, E_loc + 1] (absolute rows), demand, sorted_assign,
    assign_pos, x_sorted)."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    o = dict(out or {})
    n = T * k
    o.setdefault("round_counts", torch.empty((rounds, num_local_experts), dtype=torch.int32, device=dev))
    o.setdefault("round_offsets", torch.empty((rounds, num_local_experts + 1), dtype=torch.int32, device=dev))
    o.setdefault("demand", torch.empty(num_local_experts, dtype=torch.int32, device=dev))
    o.setdefault("sorted_assign", torch.empty(max(n, 1), dtype=torch.int32, device=dev))
    o.setdefault("assign_pos", torch.empty(max(n, 1), dtype=torch.int32, device=dev))
    hidden, dtype = 0, MOE_BF16
    if x is not None:
        dtype = _code(x.dtype)
        _dev(x, x.dtype, "x")
        if x.dim() != 2 or x.shape[0] < T:
            raise MoeError(f"x must be [>= {T}, hidden], got {tuple(x.shape)}")
        hidden = x.shape[1]
        o.setdefault("x_sorted", torch.empty((max(n, 1), hidden), dtype=x.dtype, device=dev))
        _dev(o["x_sorted"], x.dtype, "x_sorted")
        if o["x_sorted"].dim() != 2 or o["x_sorted"].shape[1] != hidden or o["x_sorted"].shape[0] < n:
            raise MoeError(f"x_sorted must be [>= {n}, {hidden}], got {tuple(o['x_sorted'].shape)}")
    else:
        o["x_sorted"] = None
    for name, need_n in (("round_counts", rounds * num_local_experts),
                         ("round_offsets", rounds * (num_local_experts + 1)),
                         ("demand", num_local_experts), ("sorted_assign", n), ("assign_pos", n)):
        _at_least(_dev(o[name], torch.int32, name), need_n, name)
    need = int(lib().moe_dispatch_deferred_workspace_size(T, k, num_local_experts))
    if need == 0:
        raise MoeError("moe_dispatch_deferred: unsupported sizes")
    ws = o.get("workspace")
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().moe_dispatch_deferred(_ptr(topk_ids), T, k, expert_begin, num_local_experts, int(capacity),
                                       int(rounds), _ptr(x), hidden, dtype, _ptr(o["round_counts"]),
                                       _ptr(o["round_offsets"]), _ptr(o["demand"]), _ptr(o["sorted_assign"]),
                                       _ptr(o["assign_pos"]), _ptr(o["x_sorted"]), _ptr(ws), ws.numel(),
                                       _stream(stream)), "moe_dispatch_deferred")
    return o


def moe_eplb_remap_capacity(topk_ids, replica_offsets, replica_slots, capacity, physical_ids=None,
                            workspace=None, stream=None):
    """Physical slot per routed (token, slot) with a per-replica capacity: the i-th assignment of
    logical expert e goes to its replica i // capacity (in table order), or -1 past them."""
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(replica_offsets, torch.int32, "replica_offsets")
    _dev(replica_slots, torch.int32, "replica_slots")
    T, k = topk_ids.shape
    E = replica_offsets.numel() - 1
    if E < 1:
        raise MoeError("the replica table is empty")
    if physical_ids is None:
        physical_ids = torch.empty_like(topk_ids)
    _shape(_dev(physical_ids, torch.int32, "physical_ids"), (T, k), "physical_ids")
    need = int(lib().moe_eplb_remap_capacity_workspace_size(T, k, E))
    if need == 0:
        raise MoeError("moe_eplb_remap_capacity: unsupported sizes")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=topk_ids.device)
    _check(lib().moe_eplb_remap_capacity(_ptr(topk_ids), T, k, _ptr(replica_offsets), _ptr(replica_slots), E,
                                         int(capacity), _ptr(physical_ids), _ptr(workspace), workspace.numel(),
                                         _stream(stream)), "moe_eplb_remap_capacity")
    return physical_ids


class MoELayer:
    """One GPU's share of the MoE layer with its buffers allocated once.

    forward() enqueues the four calls on the current stream and returns y;
    intermediates stay in self.buf.
    """

    def __init__(self, *, num_tokens, num_experts, top_k, num_groups, topk_groups, score_mode,
                 renormalize, expert_begin, num_local_experts, hidden, inter, dtype, device,
                 fuse_gather=True, expert_capacity=None, fp8=False, masked_capacity=None,
                 reroute_capacity=None, deferred=None):
        self.T, self.E, self.k = num_tokens, num_experts, top_k
        self.num_groups, self.topk_groups = num_groups, topk_groups
        self.score_mode, self.renormalize = score_mode, renormalize
        self.expert_begin, self.num_local = expert_begin, num_local_experts
        self.hidden, self.inter, self.dtype = hidden, inter, dtype
        self.fuse_gather = fuse_gather
        self.expert_capacity = expert_capacity
        self.fp8 = fp8   # e4m3 weights with block scales; x is quantised per row in forward()
        if fp8 and not fuse_gather:
            raise MoeError("the FP8 layer reads the token rows through sorted_assign (fuse_gather=True)")
        # masked layout: fixed slots of masked_capacity rows per local expert
        self.masked_capacity = masked_capacity
        # capacity with the next-best expert overflow policy, applied by the router
        self.reroute_capacity = reroute_capacity
        # (C, rounds): capacity with the overflow deferred to later rounds, one FFN call per round
        self.deferred = deferred
        if deferred is not None and (fp8 or masked_capacity is not None or expert_capacity is not None):
            raise MoeError("the deferred policy is a bf16 / float32 grouped layer with its own capacity")
        if masked_capacity is not None and (fp8 or expert_capacity is not None):
            raise MoeError("the masked layout is a bf16 / float32 layer with its own capacity")
        cap = num_tokens * top_k
        self.cap = cap
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.buf = dict(
            topk_ids=torch.empty((num_tokens, top_k), **i32),
            topk_weights=torch.empty((num_tokens, top_k), dtype=torch.float32, device=dev),
            counts=torch.empty(num_local_experts, **i32),
            offsets=torch.empty(num_local_experts + 1, **i32),
            sorted_assign=torch.empty(max(cap, 1), **i32),
            assign_pos=torch.empty(max(cap, 1), **i32),
        )
        if reroute_capacity is not None:
            rneed = int(lib().moe_route_reroute_workspace_size(num_tokens, num_experts, top_k, num_groups,
                                                               topk_groups))
            self.buf["reroute_ws"] = torch.empty(max(rneed, 1), dtype=torch.uint8, device=dev)
            self.buf["expert_load"] = torch.empty(num_experts, **i32)
        dneed = int(lib().moe_dispatch_workspace_size(num_tokens, top_k, num_local_experts))
        if deferred is not None:
            C, R = deferred
            dneed = int(lib().moe_dispatch_deferred_workspace_size(num_tokens, top_k, num_local_experts))
            self.buf.update(round_counts=torch.empty((R, num_local_experts), **i32),
                            round_offsets=torch.empty((R, num_local_experts + 1), **i32),
                            demand=torch.empty(num_local_experts, **i32))
        if dneed:
            self.buf["dispatch_ws"] = torch.empty(dneed, dtype=torch.uint8, device=dev)
        if masked_capacity is not None:
            rows = max(num_local_experts * int(masked_capacity), 1)
            self.buf.update(demand=torch.empty(num_local_experts, **i32),
                            slot_assign=torch.empty(rows, **i32))
            if hidden:
                self.buf["x_slots"] = torch.zeros((rows, hidden), dtype=dtype, device=dev)
                self.buf["o_slots"] = torch.zeros((rows, hidden), dtype=dtype, device=dev)
                self.buf["y"] = torch.empty((num_tokens, hidden), dtype=dtype, device=dev)
                need = int(lib().moe_expert_ffn_masked_workspace_size(
                    num_local_experts, hidden, inter, int(masked_capacity), _code(dtype)))
                if need == 0:
                    raise MoeError("unsupported FFN sizes")
                self.buf["workspace"] = torch.empty(need, dtype=torch.uint8, device=dev)
        elif hidden and fp8:
            self.buf["x_codes"] = torch.empty((num_tokens, hidden), dtype=torch.uint8, device=dev)
            self.buf["x_scales"] = torch.empty((num_tokens, hidden // 128), dtype=torch.float32, device=dev)
            self.buf["o_sorted"] = torch.empty((max(cap, 1), hidden), dtype=torch.bfloat16, device=dev)
            self.buf["y"] = torch.empty((num_tokens, hidden), dtype=torch.bfloat16, device=dev)
            need = ffn_fp8_workspace_size(num_local_experts, hidden, inter, max(cap, 1))
            if need == 0:
                raise MoeError("unsupported FFN sizes")
            self.buf["workspace"] = torch.empty(need, dtype=torch.uint8, device=dev)
        elif hidden:
            if not fuse_gather:
                self.buf["x_sorted"] = torch.empty((max(cap, 1), hidden), dtype=dtype, device=dev)
            self.buf["o_sorted"] = torch.empty((max(cap, 1), hidden), dtype=dtype, device=dev)
            self.buf["y"] = torch.empty((num_tokens, hidden), dtype=dtype, device=dev)
            need = ffn_workspace_size(num_local_experts, hidden, inter, max(cap, 1), dtype)
            if need == 0:
                raise MoeError("unsupported FFN sizes")
            self.buf["workspace"] = torch.empty(need, dtype=torch.uint8, device=dev)

    def route(self, scores, stream=None):
        b = self.buf
        if self.reroute_capacity is not None:
            return moe_route_reroute(scores, self.k, self.reroute_capacity, self.num_groups, self.topk_groups,
                                     self.renormalize, b["topk_ids"], b["topk_weights"], b["expert_load"],
                                     b["reroute_ws"], stream)[:2]
        return moe_route(scores, self.k, self.num_groups, self.topk_groups, self.score_mode,
                         self.renormalize, b["topk_ids"], b["topk_weights"], stream)

    def dispatch(self, x=None, stream=None):
        """Counting sort; also gathers x into x_sorted unless the gather is fused into the FFN."""
        b = self.buf
        if self.masked_capacity is not None:
            out = {n: b[n] for n in ("counts", "demand", "slot_assign", "assign_pos")}
            if "dispatch_ws" in b:
                out["workspace"] = b["dispatch_ws"]
            if x is not None:
                out["x_slots"] = b["x_slots"]
            return moe_dispatch_masked(b["topk_ids"], self.expert_begin, self.num_local,
                                       self.masked_capacity, x, out, stream)
        if self.deferred is not None:
            out = {n: b[n] for n in ("round_counts", "round_offsets", "demand", "sorted_assign", "assign_pos")}
            out["workspace"] = b["dispatch_ws"]
            xg = None
            if x is not None and not self.fuse_gather:
                out["x_sorted"], xg = b["x_sorted"], x
            return moe_dispatch_deferred(b["topk_ids"], self.expert_begin, self.num_local, self.deferred[0],
                                         self.deferred[1], xg, out, stream)
        out = {n: b[n] for n in ("counts", "offsets", "sorted_assign", "assign_pos")}
        if "dispatch_ws" in b:
            out["workspace"] = b["dispatch_ws"]
        if self.expert_capacity is not None:
            out["demand"] = b.setdefault("demand", torch.empty_like(b["counts"]))
        if x is not None and not self.fuse_gather:
            out["x_sorted"] = b["x_sorted"]
            return moe_dispatch(b["topk_ids"], self.expert_begin, self.num_local, x, out, stream,
                                self.expert_capacity)
        return moe_dispatch(b["topk_ids"], self.expert_begin, self.num_local, None, out, stream,
                            self.expert_capacity)

    def quantize(self, x, stream=None):
        """FP8 layer: the token rows to e4m3 codes and per-row block scales (the form the
        EP page dispatches them in)."""
        b = self.buf
        return moe_quantize_e4m3(x, b["x_codes"], b["x_scales"], stream)

    def ffn(self, w_gate_up, w_down, x=None, stream=None, w_gate_up_scales=None, w_down_scales=None):
        """The expert FFN; the FP8 layer reads the codes that quantize() left in self.buf."""
        b = self.buf
        if self.masked_capacity is not None:
            return moe_expert_ffn_masked(b["x_slots"], b["counts"], self.masked_capacity, w_gate_up, w_down,
                                         b["o_slots"], b["workspace"], stream)
        if self.fp8:
            return moe_expert_ffn_fp8(b["x_codes"], b["x_scales"], b["offsets"], w_gate_up, w_gate_up_scales, w_down,
                                      w_down_scales, row_index=b["sorted_assign"], row_index_div=self.k,
                                      row_capacity=self.cap, o_sorted=b["o_sorted"],
                                      workspace=b["workspace"], stream=stream)
        if self.deferred is not None:   # one grouped FFN call per round, over that round's offsets
            for r in range(self.deferred[1]):
                if self.fuse_gather:
                    moe_expert_ffn(x, b["round_offsets"][r], w_gate_up, w_down, row_index=b["sorted_assign"],
                                   row_index_div=self.k, row_capacity=self.cap, o_sorted=b["o_sorted"],
                                   workspace=b["workspace"], stream=stream)
                else:
                    moe_expert_ffn(b["x_sorted"], b["round_offsets"][r], w_gate_up, w_down, row_capacity=self.cap,
                                   o_sorted=b["o_sorted"], workspace=b["workspace"], stream=stream)
            return b["o_sorted"]
        if self.fuse_gather:
            return moe_expert_ffn(x, b["offsets"], w_gate_up, w_down, row_index=b["sorted_assign"],
                                  row_index_div=self.k, row_capacity=self.cap,
                                  o_sorted=b["o_sorted"], workspace=b["workspace"], stream=stream)
        return moe_expert_ffn(b["x_sorted"], b["offsets"], w_gate_up, w_down,
                              row_capacity=self.cap, o_sorted=b["o_sorted"],
                              workspace=b["workspace"], stream=stream)

    def combine(self, stream=None):
        b = self.buf
        o = b["o_slots"] if self.masked_capacity is not None else b["o_sorted"]
        return moe_combine(o, b["assign_pos"], b["topk_weights"], b["y"].dtype, b["y"], stream)

    def forward(self, scores, x=None, w_gate_up=None, w_down=None, stream=None, w_gate_up_scales=None,
                w_down_scales=None):
        self.route(scores, stream)
        self.dispatch(x, stream)
        if x is None:
            return None
        if self.fp8:
            self.quantize(x, stream)
        self.ffn(w_gate_up, w_down, x, stream, w_gate_up_scales, w_down_scales)
        return self.combine(stream)
