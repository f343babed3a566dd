"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, with a
bounds checker of every plan table the kernels read.

``tests/host_check/plan_check.cpp`` is built with g++ (no device code)
together with the library's host-only sources -- the attention plan
builder, the fragment planner, the Mamba table builder and the edge CSR --
and run over random forests, comb topologies (paths of up to 301 separate
spans), and the topologies of every synthetic workload.  It checks that each
span row, query tile, key tile, query end, 32-bit byte offset, fragment
table, Mamba predecessor / halo / successor / unit entry and edge CSR entry
stays in range, and that malformed forests are rejected.  Any sanitizer
report or failed check fails the test.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from workloads import WORKLOADS, comb, random_forest, tiny_tree

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shared_prefix_tree_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("plan.cpp", "fragments.cpp", "mamba_plan.cpp", "edge_plan.cpp")]
DRIVER = os.path.join(ROOT, "tests", "host_check", "plan_check.cpp")


def _forests():
    rng = np.random.default_rng(2024)
    out = [("tiny_tree", tiny_tree())]
    for i in range(60):
        out.append((f"random_small_{i}", random_forest(rng, max_tokens=200, max_len=20, max_depth=5)))
    for i in range(20):
        out.append((f"random_long_{i}", random_forest(rng, max_tokens=3000, max_len=700, max_depth=6,
                                                      p_new_root=0.05)))
    out += [
        ("comb_2_1_x100", comb(100, spine_len=2, leaf_len=1, tail_len=70)),
        ("comb_1_1_x255", comb(255, spine_len=1, leaf_len=1, tail_len=40)),
        ("comb_1_1_x300", comb(300, spine_len=1, leaf_len=1, tail_len=8)),
        ("comb_7_3_x40", comb(40, spine_len=7, leaf_len=3)),
    ]
    for w in WORKLOADS:
        out.append((w.name, w.topology()))
    return out


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path_factory.mktemp("host_check") / "plan_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-o", exe, DRIVER, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_plan_tables_in_range_under_sanitizers(checker, tmp_path):
    path = tmp_path / "forests.txt"
    forests = _forests()
    with open(path, "w") as f:
        for name, topo in forests:
            f.write(f"forest {name} {topo.num_segments}\n")
            for arr in (topo.parent, topo.seg_start, topo.seg_len):
                f.write(" ".join(str(int(x)) for x in arr) + "\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([checker, str(path)], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ALL OK" in r.stdout and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert f"{len(forests)} forests" in r.stdout
