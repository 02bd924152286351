"""Build-level checks of the HIP kernels (CPU only: hipcc cross-compiles for gfx950).

Every kernel of the library must keep its working set in registers: no
private (scratch) segment and no spilled registers, as reported by the
compiler's kernel metadata for gfx950.
"""
import os
import re
import subprocess
import tempfile

import pytest

from expert_routing_grouped_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")


def _kernel_metadata(src):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in B.FLAGS if f not in ("-fPIC", "-Wall")]
        cmd = [B.HIPCC, *flags, "--offload-device-only", "-S", "-o", out, os.path.join(B.CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        text = open(out).read()
    # the metadata block lists, per kernel, .name with its .private_segment_fixed_size,
    # .vgpr_spill_count and .sgpr_spill_count
    kernels = {}
    for block in re.split(r"\n  - \.", text.split("amdhsa.kernels:")[1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        vals = {k: int(v) for k, v in re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\d+)", block)}
        kernels[name.group(1)] = vals
    return kernels


@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip")])
def test_no_scratch_or_spills(src):
    kernels = _kernel_metadata(src)
    if src == "api.hip":
        return  # host-side validation and launch code only
    assert kernels, f"no kernels found in {src}"
    for name, vals in kernels.items():
        assert vals.get("private_segment_fixed_size", 0) == 0, (name, vals)
        assert vals.get("vgpr_spill_count", 0) == 0, (name, vals)
        assert vals.get("sgpr_spill_count", 0) == 0, (name, vals)
