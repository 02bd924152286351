"""The C-ABI library loads, exports every declared symbol and validates arguments on the host.

No test here touches a GPU: every call below fails validation before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

from expert_routing_grouped_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH),
                                reason="library not built (python -m expert_routing_grouped_amd.build)")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(moe._SIGNATURES) == _declared()


def test_version_and_status_strings():
    lib = moe.lib()
    assert lib.moe_abi_version() == 9
    assert moe.status_string(0) == "ok"
    assert moe.status_string(1) == "invalid argument"
    assert moe.status_string(3).startswith("workspace")
    assert moe.status_string(5).startswith("sizes exceed the fixed scratch")
    assert moe.status_string(99) == "unknown status"


def test_route_validation():
    l = moe.lib()
    R = moe.MOE_SCORE_RAW
    assert l.moe_route(None, 4, 256, 0, 8, 4, R, 1, None, None, None) == 1       # k = 0
    assert l.moe_route(None, 4, 250, 8, 8, 4, R, 1, None, None, None) == 1       # 8 does not divide 250
    assert l.moe_route(None, 4, 16, 9, 4, 2, R, 1, None, None, None) == 1        # 9 > 2 groups * 4
    assert l.moe_route(None, 4, 16, 2, 4, 5, R, 1, None, None, None) == 1        # 5 > 4 groups
    assert l.moe_route(None, 4, 16, 2, 4, 2, moe.MOE_SCORE_SOFTMAX, 0, None, None, None) == 1
    assert l.moe_route(None, 4, 16, 2, 16, 2, R, 1, None, None, None) == 1       # groups of one
    assert l.moe_route(None, 4, 2048, 8, 1, 1, R, 1, None, None, None) == 2      # E > 1024
    assert l.moe_route(None, 4, 256, 8, 8, 4, 7, 1, None, None, None) == 1       # bad score mode
    assert l.moe_route(None, 4, 256, 8, 8, 4, R, 1, None, None, None) == 1       # NULL pointers
    assert l.moe_route(None, 0, 256, 8, 8, 4, R, 1, None, None, None) == 0       # T = 0: no-op


def test_route_reroute_validation():
    l = moe.lib()
    p = ctypes.c_void_p(256)
    W = (p, 1 << 30, None)
    # (scores, T, E, k, groups, topk_groups, renorm, C, ids, weights, load, ws, ws_bytes, stream)
    assert l.moe_route_reroute(p, 4, 256, 8, 8, 4, 1, -1, p, p, None, *W) == 1    # C < 0
    assert l.moe_route_reroute(p, 4, 250, 8, 8, 4, 1, 10, p, p, None, *W) == 1    # groups
    assert l.moe_route_reroute(p, 4, 2048, 8, 1, 1, 1, 10, p, p, None, *W) == 2   # E > 1024
    assert l.moe_route_reroute(None, 4, 256, 8, 8, 4, 1, 10, p, p, None, *W) == 1  # NULL scores
    assert l.moe_route_reroute(p, 4, 256, 8, 8, 4, 1, 10, p, p, None, p, 16, None) == 3   # small ws
    assert l.moe_route_reroute(None, 0, 256, 8, 8, 4, 1, 10, None, None, None, None, 0, None) == 0
    assert l.moe_route_reroute_workspace_size(512, 256, 8, 8, 4) > 512 * 16 * 8
    assert l.moe_route_reroute_workspace_size(512, 250, 8, 8, 4) == 0


def test_dispatch_validation():
    l = moe.lib()
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    W = (None, 0, None)       # no workspace, default stream
    assert l.moe_dispatch(None, 4, 0, 0, 8, None, 0, 1, p, p, p, p, None, *W) == 1
    assert l.moe_dispatch(p, 4, 8, 0, 0, None, 0, 1, p, p, p, p, None, *W) == 1
    assert l.moe_dispatch(p, 4, 8, 0, 1025, None, 0, 1, p, p, p, p, None, *W) == 2   # > 1024 local
    assert l.moe_dispatch(p, 4, 8, 0, 8, p, 0, 1, p, p, p, p, None, *W) == 1      # x without x_sorted
    assert l.moe_dispatch(p, 4, 8, 0, 8, p, 12, 1, p, p, p, p, p, *W) == 1         # hidden % 8
    assert l.moe_dispatch(p, 4, 8, 0, 8, ctypes.c_void_p(8), 16, 1, p, p, p, p, p, *W) == 1  # unaligned
    assert l.moe_dispatch(p, 4, 8, 0, 8, None, 0, 5, p, p, p, p, None, *W) == 1    # bad dtype
    assert l.moe_dispatch(None, 4, 8, 0, 8, None, 0, 1, p, p, p, p, None, *W) == 1 # NULL ids
    # large T*k needs a workspace of one int per (2048-assignment block, local expert)
    assert l.moe_dispatch_workspace_size(1024, 8, 32) == 0
    # 65536 assignments: 64 blocks of 1024, a [blocks][experts] table plus one row of totals
    assert l.moe_dispatch_workspace_size(8192, 8, 32) == (64 + 1) * 32 * 4
    assert l.moe_dispatch(p, 8192, 8, 0, 32, None, 0, 1, p, p, p, p, None, None, 0, None) == 3
    assert l.moe_dispatch(p, 8192, 8, 0, 32, None, 0, 1, p, p, p, p, None, p, 100, None) == 3


def test_dispatch_capacity_validation():
    l = moe.lib()
    p = ctypes.c_void_p(16)
    W = (None, 0, None)
    # (ids, T, k, begin, nloc, capacity, x, hidden, dtype, counts, offsets, demand, sorted, pos, x_sorted, ws...)
    assert l.moe_dispatch_capacity(p, 4, 8, 0, 8, -1, None, 0, 1, p, p, None, p, p, None, *W) == 1
    assert l.moe_dispatch_capacity(p, 4, 0, 0, 8, 10, None, 0, 1, p, p, None, p, p, None, *W) == 1
    assert l.moe_dispatch_capacity(p, 4, 8, 0, 2000, 10, None, 0, 1, p, p, None, p, p, None, *W) == 2
    assert l.moe_dispatch_capacity(None, 4, 8, 0, 8, 10, None, 0, 1, p, p, None, p, p, None, *W) == 1
    assert l.moe_dispatch_capacity(p, 8192, 8, 0, 32, 10, None, 0, 1, p, p, p, p, p, None, *W) == 3


def test_expert_capacity_is_exact():
    """moe_expert_capacity (a host function) against the oracle's exact-rational ceiling: the
    page's example (T = 5600, k = 16, E = 896, c = 1.2 -> 120) and a case where binary floating
    point lands above the integer (T = 400, k = 1, E = 8, c = 1.1 -> 55)."""
    import math
    from fractions import Fraction

    import oracle
    for T, k, E, c in ((5600, 16, 896, "1.2"), (400, 1, 8, "1.1"), (4096, 8, 256, "1"),
                       (1, 1, 1000, "0.5"), (0, 8, 256, "1.25"), (8192, 8, 256, "2.75"),
                       (12345, 7, 333, "1.2345"), (100, 3, 7, "0")):
        f = Fraction(c)
        assert moe.moe_expert_capacity(T, k, E, f.numerator, f.denominator) == \
            oracle.expert_capacity(T, k, E, c)
    assert math.ceil(1.1 * 400 * 1 / 8) == 56      # the float product the exact form avoids
    l = moe.lib()
    out = ctypes.c_int32(0)
    assert l.moe_expert_capacity(10, 1, 1, 1, 0, ctypes.byref(out)) == 1      # den = 0
    assert l.moe_expert_capacity(10, 0, 1, 1, 1, ctypes.byref(out)) == 1      # k = 0
    assert l.moe_expert_capacity(10, 1, 1, -1, 1, ctypes.byref(out)) == 1     # c < 0
    assert l.moe_expert_capacity(10, 1, 1, 1, 1, None) == 1                   # NULL out
    assert l.moe_expert_capacity(1 << 30, 8, 1, 1, 1, ctypes.byref(out)) == 2  # T k >= 2^31
    assert l.moe_expert_capacity(1 << 20, 1024, 1, 3, 1, ctypes.byref(out)) == 2  # C >= 2^31


def test_masked_validation_and_workspace():
    l = moe.lib()
    p = ctypes.c_void_p(256)
    W = (None, 0, None)
    # (ids, T, k, begin, nloc, C, x, hidden, dtype, counts, demand, slot_assign, pos, x_slots, ws...)
    assert l.moe_dispatch_masked(p, 4, 8, 0, 8, -1, None, 0, 1, p, None, p, p, None, *W) == 1   # C < 0
    assert l.moe_dispatch_masked(p, 4, 8, 0, 8, 4, None, 0, 1, None, None, p, p, None, *W) == 1  # counts
    assert l.moe_dispatch_masked(p, 4, 8, 0, 8, 4, None, 0, 1, p, None, None, p, None, *W) == 1  # slots
    assert l.moe_dispatch_masked(p, 4, 8, 0, 1024, 1 << 21, None, 0, 1, p, None, p, p, None, *W) == 2
    assert l.moe_dispatch_masked(p, 8192, 8, 0, 32, 4, None, 0, 1, p, None, p, p, None, *W) == 3
    # FFN: workspace = compact offsets + row index + compact outputs + the FFN's own workspace
    need = l.moe_expert_ffn_masked_workspace_size(8, 7168, 2048, 32, 1)
    assert need >= 8 * 32 * 7168 * 2 + l.moe_expert_ffn_workspace_size(8, 7168, 2048, 8 * 32, 1)
    assert l.moe_expert_ffn_masked_workspace_size(8, 7000, 2048, 32, 1) == 0
    assert l.moe_expert_ffn_masked_workspace_size(8, 7168, 2048, -1, 1) == 0
    args = [p, p, 32, p, p, 8, 7168, 2048, 1, p]
    assert l.moe_expert_ffn_masked(*args, p, 16, None) == 3                      # small workspace
    assert l.moe_expert_ffn_masked(p, None, 32, p, p, 8, 7168, 2048, 1, p, p, need, None) == 1   # counts
    assert l.moe_expert_ffn_masked(p, p, -2, p, p, 8, 7168, 2048, 1, p, p, need, None) == 1
    assert l.moe_expert_ffn_masked(p, p, 32, p, p, 8, 7000, 2048, 1, p, p, need, None) == 2


def test_ffn_validation_and_workspace():
    l = moe.lib()
    p = ctypes.c_void_p(256)
    assert l.moe_expert_ffn_workspace_size(8, 7168, 2048, 4096, 1) >= 4096 * 2048 * 2
    assert l.moe_expert_ffn_workspace_size(8, 7000, 2048, 4096, 1) == 0     # hidden % 256
    assert l.moe_expert_ffn_workspace_size(8, 7168, 100, 4096, 1) == 0      # inter % 64
    assert l.moe_expert_ffn_workspace_size(0, 7168, 2048, 4096, 1) == 0
    assert l.moe_expert_ffn(p, None, 1, p, p, p, 8, 7000, 2048, 64, 1, p, p, 1 << 30, None) == 2
    assert l.moe_expert_ffn(p, None, 1, None, p, p, 8, 7168, 2048, 64, 1, p, p, 1 << 30, None) == 1
    assert l.moe_expert_ffn(p, p, 0, p, p, p, 8, 7168, 2048, 64, 1, p, p, 1 << 30, None) == 1  # div 0
    assert l.moe_expert_ffn(p, None, 1, p, p, p, 8, 7168, 2048, 64, 1, p, p, 16, None) == 3   # small ws
    assert l.moe_expert_ffn(p, None, 1, p, p, p, 8, 7168, 2048, 64, 1, p, None, 1 << 30, None) == 3
    assert l.moe_expert_ffn(p, None, 1, p, p, p, 8000, 256, 64, 64, 0, p, p, 1 << 30, None) == 2
    # the allocation-free variant validates the same way, and refuses sizes whose workspace
    # exceeds its fixed 64 MiB scratch before it looks anything up on a device
    assert l.moe_expert_ffn_noalloc(p, None, 1, p, p, p, 8, 7000, 2048, 64, 1, p, None) == 2
    assert l.moe_expert_ffn_noalloc(p, None, 1, None, p, p, 8, 7168, 2048, 64, 1, p, None) == 1
    assert l.moe_expert_ffn_noalloc(p, p, 0, p, p, p, 8, 7168, 2048, 64, 1, p, None) == 1
    assert l.moe_expert_ffn_workspace_size(8, 7168, 2048, 65536, 1) > moe.NOALLOC_SCRATCH_BYTES
    assert l.moe_expert_ffn_noalloc(p, p, 8, p, p, p, 32, 7168, 2048, 65536, 1, p, None) == 5
    assert l.moe_expert_ffn_workspace_size(8, 7168, 2048, 4096, 1) <= moe.NOALLOC_SCRATCH_BYTES
    assert l.moe_expert_ffn_workspace_size(256, 7168, 64, 4096, 1) <= moe.NOALLOC_SCRATCH_BYTES


def test_fp8_validation_and_workspace():
    l = moe.lib()
    p = ctypes.c_void_p(256)
    f = ctypes.cast(p, ctypes.POINTER(ctypes.c_float))
    # quantiser: (x, rows, cols, dtype, codes, scales, stream)
    assert l.moe_quantize_e4m3(p, 4, 100, 1, p, f, None) == 1        # cols % 128
    assert l.moe_quantize_e4m3(p, 4, 256, 7, p, f, None) == 1        # bad dtype
    assert l.moe_quantize_e4m3(None, 4, 256, 1, p, f, None) == 1     # NULL x
    assert l.moe_quantize_e4m3(ctypes.c_void_p(8), 4, 256, 1, p, f, None) == 1   # unaligned
    assert l.moe_quantize_e4m3(None, 0, 256, 1, None, None, None) == 0           # no rows: no-op
    # FFN: workspace = h in float32, h codes, h scales (each 256-byte aligned)
    assert l.moe_expert_ffn_fp8_workspace_size(8, 7168, 2048, 4096) == \
        4096 * 2048 * 4 + 4096 * 2048 + 4096 * 16 * 4
    assert l.moe_expert_ffn_fp8_workspace_size(8, 7168 + 256, 2048, 4096) == 0   # hidden % 512
    assert l.moe_expert_ffn_fp8_workspace_size(8, 7168, 2048 + 128, 4096) == 0   # inter % 256
    assert l.moe_expert_ffn_fp8_workspace_size(2000, 7168, 2048, 4096) == 0      # E_loc > 1024
    W = (p, 1 << 30, None)
    args = lambda **kw: [kw.get("x", p), kw.get("xs", f), kw.get("ri", None), kw.get("div", 1),
                         kw.get("off", p), kw.get("wg", p), kw.get("wgs", f), kw.get("wd", p),
                         kw.get("wds", f), kw.get("nloc", 8), kw.get("d", 7168), kw.get("I", 2048),
                         kw.get("cap", 64), kw.get("o", p)]
    assert l.moe_expert_ffn_fp8(*args(d=7000), *W) == 2
    assert l.moe_expert_ffn_fp8(*args(off=None), *W) == 1
    assert l.moe_expert_ffn_fp8(*args(wgs=None), *W) == 1
    assert l.moe_expert_ffn_fp8(*args(ri=p, div=0), *W) == 1
    assert l.moe_expert_ffn_fp8(*args(o=None), *W) == 1
    assert l.moe_expert_ffn_fp8(*args(x=ctypes.c_void_p(264)), *W) == 1          # unaligned codes
    assert l.moe_expert_ffn_fp8(*args(), p, 16, None) == 3                       # small workspace
    assert l.moe_expert_ffn_fp8(*args(cap=300000), *W) == 2                      # h offsets >= 2^31


def test_combine_validation():
    l = moe.lib()
    p = ctypes.c_void_p(256)
    assert l.moe_combine(p, p, p, 4, 0, 7168, 1, 1, p, None) == 1
    assert l.moe_combine(p, p, p, 4, 8, 7164, 1, 1, p, None) == 1
    assert l.moe_combine(p, p, p, 4, 100, 7168, 1, 1, p, None) == 2
    assert l.moe_combine(None, p, p, 4, 8, 7168, 1, 1, p, None) == 1
    assert l.moe_combine(p, p, p, 0, 8, 7168, 1, 1, p, None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(moe.MoeError):
        moe.lib()


def test_deferred_and_replica_capacity_validation():
    """The deferred dispatch and the capacity-aware replica choice: workspace sizes and argument
    checks (every call below fails validation before anything is enqueued)."""
    l = moe.lib()
    p = ctypes.c_void_p(256)
    ws = l.moe_dispatch_deferred_workspace_size(512, 8, 8)
    assert ws >= (8 + 9 + 4096) * 4
    assert l.moe_dispatch_deferred_workspace_size(70001, 8, 256) > l.moe_dispatch_workspace_size(70001, 8, 256)
    assert l.moe_dispatch_deferred_workspace_size(512, 8, 1025) == 0
    assert l.moe_dispatch_deferred_workspace_size(-1, 8, 8) == 0
    args = lambda **kw: [kw.get("ids", p), 512, 8, 0, 8, kw.get("C", 20), kw.get("R", 2), None, 0, 1,
                         kw.get("rc", p), kw.get("ro", p), None, p, p, None, kw.get("ws", p),
                         kw.get("wsb", ws), None]
    assert l.moe_dispatch_deferred(*args(C=-1)) == 1
    assert l.moe_dispatch_deferred(*args(R=0)) == 1
    assert l.moe_dispatch_deferred(*args(rc=None)) == 1
    assert l.moe_dispatch_deferred(*args(ids=None)) == 1
    assert l.moe_dispatch_deferred(*args(wsb=ws - 1)) == 3
    assert l.moe_dispatch_deferred(*args(ws=None)) == 3
    bad_ids = args()
    bad_ids[4] = 1025                                                     # local experts past the limit
    assert l.moe_dispatch_deferred(*bad_ids) == 2
    rws = l.moe_eplb_remap_capacity_workspace_size(512, 8, 256)
    assert rws >= (256 + 257 + 2 * 4096) * 4
    assert l.moe_eplb_remap_capacity_workspace_size(512, 8, 1025) == 0
    assert l.moe_eplb_remap_capacity(p, 512, 8, p, p, 256, -1, p, p, rws, None) == 1
    assert l.moe_eplb_remap_capacity(p, 512, 8, None, p, 256, 4, p, p, rws, None) == 1
    assert l.moe_eplb_remap_capacity(p, 512, 8, p, p, 256, 4, p, p, rws - 1, None) == 3
    assert l.moe_eplb_remap_capacity(p, 512, 8, p, p, 1025, 4, p, p, rws, None) == 2
    assert l.moe_eplb_remap_capacity(None, 0, 8, None, None, 256, 4, None, None, 0, None) == 0   # T = 0: no-op
