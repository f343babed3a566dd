"""C-ABI library: loads, exports every declared symbol, and its host plan
logic (validation, spans, tiles) agrees with the oracle's definitions.

No compute call is made here (no GPU needed): plans are built host-only.
"""

import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import shared_prefix_tree_amd as sp
from shared_prefix_tree_amd import binding as b
from workloads import WORKLOADS, Topology, random_forest, tiny_tree

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tree_attn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = sp.library()
    declared = declared_functions()
    assert declared == sorted(b.SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r" T (tree_attn_\w+)", nm.stdout))
    assert set(declared) <= exported


def plan_tables(topo):
    p = sp.Plan.from_topology(topo, device=False)
    return p, {
        "span_ptr": p.export(b.EXPORT_SPAN_PTR),
        "spans": p.export(b.EXPORT_SPANS),
        "qt": p.export(b.EXPORT_Q_TILES),
        "kt": p.export(b.EXPORT_KV_TILES),
        "depth": p.export(b.EXPORT_SEG_DEPTH),
        "prefix": p.export(b.EXPORT_SEG_PREFIX),
        "end": p.export(b.EXPORT_SEG_END),
    }


def topologies():
    rng = np.random.default_rng(0)
    tops = [random_forest(rng, max_tokens=300, max_len=70, max_depth=5) for _ in range(15)]
    tops += [tiny_tree(), Topology([-1], [0], [1]), Topology([-1, -1, -1], [0, 1, 2], [1, 1, 1])]
    return tops


@pytest.mark.parametrize("idx", range(18))
def test_plan_spans_cover_exactly_the_visible_sets(idx):
    topo = topologies()[idx]
    p, t = plan_tables(topo)
    info = p.info()
    assert info["pairs"] == oracle.pairs(topo)
    assert info["total_tokens"] == topo.total_tokens
    assert info["on_device"] == 0
    seg_of = np.repeat(np.arange(topo.num_segments), topo.seg_len)
    for s in range(topo.num_segments):
        spans = t["spans"][t["span_ptr"][s] : t["span_ptr"][s + 1]]
        # merged spans are disjoint, in virtual order, and not mergeable further
        virt = 0
        for k, (phys, ln, v, _) in enumerate(spans):
            assert v == virt and ln >= 1
            if k:
                assert spans[k - 1][0] + spans[k - 1][1] != phys
            virt += ln
        assert virt == t["prefix"][s] + topo.seg_len[s]
        path = np.concatenate([np.arange(ph, ph + ln) for ph, ln, _, _ in spans])
        # the path truncated at each query's position is exactly V(i)
        for i in range(topo.seg_start[s], topo.seg_start[s] + topo.seg_len[s]):
            pos = t["prefix"][s] + (i - topo.seg_start[s])
            assert np.array_equal(path[: pos + 1], oracle.visible_tokens(topo, i))
    np.testing.assert_array_equal(t["end"], oracle.subtree_end(topo))
    parent = topo.parent
    for s in range(topo.num_segments):
        assert t["depth"][s] == len(oracle.ancestors(parent, s))
    # query tiles: every token once, within one segment, longest key range first
    qt = t["qt"]
    cover = np.zeros(topo.total_tokens, dtype=int)
    for q0, nq, seg, pos0 in qt:
        assert 1 <= nq <= 32
        assert np.all(seg_of[q0 : q0 + nq] == seg)
        assert pos0 == oracle.position_in_sequence(topo, q0)
        cover[q0 : q0 + nq] += 1
    assert np.all(cover == 1)
    work = qt[:, 3] + qt[:, 1]
    assert np.all(work[:-1] >= work[1:])
    # key tiles: every token once; [k0, qend) is exactly the queries seeing k0
    kt = t["kt"]
    cover[:] = 0
    m = oracle.visible_mask(topo)
    for k0, nk, seg, qend in kt:
        assert 1 <= nk <= 64
        assert np.all(seg_of[k0 : k0 + nk] == seg)
        cover[k0 : k0 + nk] += 1
        for j in range(k0, k0 + nk):
            seers = np.nonzero(m[:, j])[0]
            assert seers.min() == j and seers.max() == qend - 1 and len(seers) == qend - j
    assert np.all(cover == 1)
    rng_ = kt[:, 3] - kt[:, 0]
    assert np.all(rng_[:-1] >= rng_[1:])


def test_workload_plans_match_oracle_pairs():
    for w in WORKLOADS:
        topo = w.topology()
        info = sp.Plan.from_topology(topo, device=False).info()
        assert info["pairs"] == oracle.pairs(topo), w.name
        assert info["max_path_len"] == max(
            oracle.position_in_sequence(topo, int(s + n - 1)) + 1 for s, n in zip(topo.seg_start, topo.seg_len)
        )


BAD = [
    ("empty", [], [], []),
    ("zero_length", [-1, 0], [0, 4], [4, 0]),
    ("negative_length", [-1], [0], [-3]),
    ("gap", [-1, 0], [0, 5], [4, 2]),
    ("not_from_zero", [-1], [1], [4]),
    ("parent_after_self", [-1, 2, 0], [0, 1, 2], [1, 1, 1]),
    ("parent_self", [-1, 1], [0, 1], [1, 1]),
    ("parent_below_minus_one", [-2], [0], [1]),
    ("not_dfs", [-1, 0, 1, 0, 2], [0, 1, 2, 3, 4], [1, 1, 1, 1, 1]),
    ("sibling_of_closed", [-1, 0, 0, 1], [0, 1, 2, 3], [1, 1, 1, 1]),
]


@pytest.mark.parametrize("name,parent,start,length", BAD, ids=[x[0] for x in BAD])
def test_plan_rejects_malformed_topologies(name, parent, start, length):
    with pytest.raises(sp.TreeAttnError) as e:
        sp.Plan(parent, start, length, device=False)
    assert e.value.code == b.INVALID_ARGUMENT
    assert str(e.value)


def test_plan_rejects_too_many_tokens():
    n = 1 << 16
    with pytest.raises(sp.TreeAttnError) as e:
        sp.Plan(np.full(n, -1), np.arange(n, dtype=np.int64) * (1 << 15), np.full(n, 1 << 15), device=False)
    assert e.value.code == b.INVALID_ARGUMENT


def test_null_arguments_are_rejected_without_a_device():
    import ctypes

    lib = sp.library()
    assert lib.tree_attn_plan_destroy(None) == b.OK
    assert lib.tree_attn_plan_info(None, None) == b.INVALID_ARGUMENT
    assert lib.tree_attn_last_error().decode()
    shape = b.Shape(4, 1, 1, 64, b.FP32, 0.0)
    # host-only plan: fwd/bwd refuse before touching any device memory
    p = sp.Plan([-1], [0], [4], device=False)
    rc = lib.tree_attn_fwd(None, None, None, p.handle, ctypes.byref(shape), None, None, None)
    assert rc == b.INVALID_ARGUMENT
    one = ctypes.c_void_p(256)  # never dereferenced: rejected before any launch
    rc = lib.tree_attn_fwd(one, one, one, p.handle, ctypes.byref(shape), one, one, None)
    assert rc == b.INVALID_ARGUMENT and "host-only" in lib.tree_attn_last_error().decode()
    # two [Hq, T] float32 arrays rounded up to 256 bytes, then two 64-byte counter blocks
    assert lib.tree_attn_bwd_workspace_bytes(p.handle, ctypes.byref(shape)) == 256 + 128
    rc = lib.tree_attn_bwd(*([one] * 6), p.handle, ctypes.byref(shape), one, one, one, one, 1 << 20, None)
    assert rc == b.INVALID_ARGUMENT


def test_backward_stages_reject_null_inputs_before_launch():
    """Every backward stage checks each pointer it reads (lse included) before
    any launch; a host-only plan would be rejected later, so a NULL pointer
    must be what is reported."""
    import ctypes

    lib = sp.library()
    p = sp.Plan([-1], [0], [4], device=False)
    shape = b.Shape(4, 1, 1, 64, b.FP32, 0.0)
    one = ctypes.c_void_p(256)  # never dereferenced
    ws = ctypes.c_size_t(1 << 20)
    assert lib.tree_attn_bwd_rowstat(one, None, one, p.handle, ctypes.byref(shape), one, ws, None) == b.INVALID_ARGUMENT
    assert "NULL" in lib.tree_attn_last_error().decode()
    assert lib.tree_attn_bwd_rowstat(None, one, one, p.handle, ctypes.byref(shape), one, ws, None) == b.INVALID_ARGUMENT
    assert lib.tree_attn_bwd_rowstat(one, one, None, p.handle, ctypes.byref(shape), one, ws, None) == b.INVALID_ARGUMENT
    args = [one] * 5
    for i in range(5):  # q, k, v, lse, dout
        a = list(args)
        a[i] = None
        assert lib.tree_attn_bwd_dkdv(*a, p.handle, ctypes.byref(shape), one, one, one, ws, None) == b.INVALID_ARGUMENT
        assert "NULL" in lib.tree_attn_last_error().decode()
        assert lib.tree_attn_bwd_dq(*a, p.handle, ctypes.byref(shape), one, one, ws, None) == b.INVALID_ARGUMENT
    assert lib.tree_attn_bwd_dkdv(*args, p.handle, ctypes.byref(shape), None, one, one, ws, None) == b.INVALID_ARGUMENT
    assert lib.tree_attn_bwd_dq(*args, p.handle, ctypes.byref(shape), None, one, ws, None) == b.INVALID_ARGUMENT
    # with every pointer present the host-only plan is what is reported
    assert lib.tree_attn_bwd_rowstat(one, one, one, p.handle, ctypes.byref(shape), one, ws, None) == b.INVALID_ARGUMENT
    assert "host-only" in lib.tree_attn_last_error().decode()


@pytest.mark.parametrize("src,tgt,T,V,frag", [
    ([0, 5], [1, 2], 5, 10, "edge 1 has source 5"),
    ([0, 1], [1, 10], 5, 10, "edge 1 has source 1 / sampled token 10"),
    ([0, -1], [1, 2], 5, 10, "edge 1"),
    ([], [], 5, 10, "need >= 1 edge"),
])
def test_edge_plan_rejects_bad_edges_without_a_device(src, tgt, T, V, frag):
    with pytest.raises(b.TreeAttnError, match=frag):
        sp.EdgePlan(np.array(src, np.int32), np.array(tgt, np.int32), T, V)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """There is no CPU fallback: without the built library every entry point
    raises instead of computing something else."""
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        b.library()
    with pytest.raises(RuntimeError, match="no fallback"):
        sp.Plan([-1], [0], [4], device=False)


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "shared_prefix_tree_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), f
                assert "oracle/" not in src, f


def test_mamba_calls_reject_a_host_only_plan_without_a_device():
    plan = sp.MambaPlan([-1, 0], [0, 4], [4, 4], device=False)
    lib = sp.library()
    rc = lib.tree_attn_conv_fwd(None, None, None, 8, 4, 4, plan.handle, None, None)
    assert rc == b.INVALID_ARGUMENT
    assert "host-only" in lib.tree_attn_last_error().decode()
