"""The library's host planning code (EPLB placement, exact capacity) built on its own with g++
under the address and undefined-behaviour sanitizers, run on the EPLB page's placements and on
random loads with ties and zeros, and compared with the oracle (CPU only)."""
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import eplb
from expert_routing_grouped_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_routing_grouped_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "host_plan_driver.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("san") / "host_plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(CSRC, "host_plan.cpp"), DRIVER, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout.splitlines()


def placement_case(load, G, nodes, gpus, phys, hier):
    return "P %d %d %d %d %d %d %s" % (len(load), G, nodes, gpus, phys, int(hier),
                                       " ".join(repr(float(v)) for v in load))


def parse_placement(line, E, phys):
    head, offs, slots = line.split("|")
    vals = [int(v) for v in head.split()[1:]]
    return vals[0], np.array(vals[1:]), np.array([int(v) for v in offs.split()]), \
        np.array([int(v) for v in slots.split()])


def cases():
    scores = W.page_simulation_scores()
    ids, _ = oracle.route_grouped(scores, 8, 8, 4)
    page_load = np.bincount(ids.ravel(), minlength=256).astype(float)
    out = [(page_load, 8, n, g, p, h) for n, g, p in ((4, 32, 288), (8, 64, 320)) for h in (False, True)]
    rng = np.random.default_rng(3)
    for _ in range(12):
        G = int(rng.choice([1, 2, 4, 8]))
        E = G * int(rng.integers(1, 9))
        nodes = int(rng.choice([n for n in (1, 2, 4) if G % n == 0]))
        gpus = nodes * int(rng.integers(1, 4))
        per_node_extra = int(rng.integers(0, 4))
        phys = E + nodes * per_node_extra * (gpus // nodes)
        phys += (-phys) % gpus
        load = rng.integers(0, 5, E).astype(float)          # ties and zeros
        hier = bool(rng.integers(0, 2)) and E % nodes == 0 and phys % nodes == 0 and \
            (phys // nodes) % (gpus // nodes) == 0
        out.append((load, G, nodes, gpus, phys, hier))
    return out


def test_placement_under_sanitizers_matches_oracle(driver):
    cs = cases()
    lines = run(driver, [placement_case(*c) for c in cs])
    assert len(lines) == len(cs)
    for (load, G, nodes, gpus, phys, hier), line in zip(cs, lines):
        n, p2l, offs, slots = parse_placement(line, len(load), phys)
        assert n == phys
        ref = [e for g in eplb.place(load, G, nodes, gpus, phys, hier) for e in g]
        assert p2l.tolist() == ref
        # the replica table lists each expert's slots in ascending order
        E = len(load)
        assert offs[0] == 0 and offs[-1] == phys
        for e in range(E):
            got = slots[offs[e]:offs[e + 1]].tolist()
            assert got == [s for s in range(phys) if ref[s] == e]


def test_capacity_under_sanitizers(driver):
    cs = [(5600 * 16, "1.2", 896), (400, "1.1", 8), (4096 * 8, "1", 256), (0, "1.25", 256),
          ((1 << 31) - 1, "2147483647", 1), (12345 * 7, "1.2345", 333)]
    lines = run(driver, ["C %d %d %d %d" % (tk, Fraction(c).numerator, Fraction(c).denominator, E)
                         for tk, c, E in cs])
    for (tk, c, E), line in zip(cs, lines):
        assert int(line.split()[1]) == -(-Fraction(c) * tk // E)
