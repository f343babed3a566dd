"""Bounded fragment planning with ancestor repetition (host only).

Issue "Shared-prefix training with context parallelism for exact agent
trajectories", section "Describe the solution you'd like": fragments are
size-bounded, and ancestor segments may be duplicated in several of them.
The oracle
(``oracle.fragment``) is pinned by a hand-worked case and by the property
that makes the repetition exact -- every owned token sees, mapped back to
source tokens, exactly its visible set in the source forest; the library's
``tree_attn_fragment`` must then match the oracle table for table.
"""

import json
import os

import numpy as np
import pytest

import oracle
import shared_prefix_tree_amd.binding as b
from workloads import Topology, agent_tree, random_forest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fragments_small.json")


def check_exact_repetition(topo, frags, bound):
    """Invariants that pin any planner: bound, ownership once, DFS forests,
    and visible sets preserved for every owned token."""
    T = topo.total_tokens
    owned = np.zeros(T, int)
    for fr in frags:
        par, ln, src, own = (np.asarray(fr[k]) for k in ("parent", "seg_len", "source", "owner"))
        assert len(src) == int(ln.sum()) <= bound
        st = np.concatenate([[0], np.cumsum(ln)[:-1]]).astype(np.int32)
        sub = Topology(par.tolist(), st.tolist(), ln.tolist())
        b.Plan(sub.parent, sub.seg_start, sub.seg_len, device=False).close()  # a valid DFS forest
        for i in np.nonzero(own)[0]:
            owned[src[i]] += 1
            got = sorted(src[oracle.visible_tokens(sub, int(i))].tolist())
            want = sorted(oracle.visible_tokens(topo, int(src[i])).tolist())
            assert got == want
        # a copy is a copy of its own source token's row: sources of a segment are consecutive
        for s in range(len(ln)):
            seg_src = src[st[s]:st[s] + ln[s]]
            assert np.array_equal(seg_src, np.arange(seg_src[0], seg_src[0] + ln[s]))
    assert np.array_equal(owned, np.ones(T, int))


def test_oracle_matches_the_hand_worked_case():
    g = json.load(open(GOLDEN))
    f = g["forest"]
    got = oracle.fragment(f["parent"], f["seg_start"], f["seg_len"], g["max_tokens"])
    assert got == g["fragments"]
    topo = Topology(f["parent"], f["seg_start"], f["seg_len"])
    check_exact_repetition(topo, got, g["max_tokens"])


@pytest.mark.parametrize("seed", [51, 52, 53, 54])
def test_oracle_keeps_every_visible_set(seed):
    rng = np.random.default_rng(seed)
    topo = random_forest(rng, max_tokens=260, max_len=40, max_depth=4, p_new_root=0.2)
    longest = max(len(oracle.visible_tokens(topo, i)) for i in range(topo.total_tokens))
    for bound in (longest, longest + 7, 2 * longest + 3):
        frags = oracle.fragment(topo.parent, topo.seg_start, topo.seg_len, bound)
        check_exact_repetition(topo, frags, bound)


def test_library_matches_the_oracle_table_for_table():
    g = json.load(open(GOLDEN))
    f = g["forest"]
    frags, info = b.fragment(f["parent"], f["seg_start"], f["seg_len"], g["max_tokens"])
    assert [{k: fr[k].tolist() for k in ("parent", "seg_len", "source", "owner")} for fr in frags] == g["fragments"]
    assert (info["num_fragments"], info["source_tokens"], info["fragment_tokens"]) == (3, 29, 42)
    for seed in (61, 62, 63):
        rng = np.random.default_rng(seed)
        topo = random_forest(rng, max_tokens=900, max_len=120, max_depth=5, p_new_root=0.1)
        longest = max(len(oracle.visible_tokens(topo, i)) for i in range(topo.total_tokens))
        for bound in (longest, longest + 1, 3 * longest):
            ref = oracle.fragment(topo.parent, topo.seg_start, topo.seg_len, bound)
            got, info = b.fragment(topo.parent, topo.seg_start, topo.seg_len, bound)
            assert len(got) == len(ref) == info["num_fragments"]
            for a, r in zip(got, ref):
                for k in ("parent", "seg_len", "source", "owner"):
                    assert a[k].tolist() == r[k], (seed, bound, k)
            check_exact_repetition(topo, got, bound)


def test_library_rejects_a_path_longer_than_the_bound():
    import ctypes

    lib = b.library()
    p, pp = b._i32([-1, 0])
    s, sp = b._i32([0, 10])
    n, np_ = b._i32([10, 5])
    h = ctypes.c_void_p()
    for bound in (14, 0, -3):
        assert lib.tree_attn_fragment(pp, sp, np_, 2, bound, ctypes.byref(h)) == b.INVALID_ARGUMENT
        assert "tree_attn_fragment" in lib.tree_attn_last_error().decode()
    assert lib.tree_attn_fragment(pp, sp, np_, 2, 15, ctypes.byref(h)) == b.OK
    lib.tree_attn_fragments_destroy(h)


def test_agent_tree_duplication_at_the_fragment_bound():
    """The pages' metric for this step is the token count before and after
    fragmentation; on the 65,536-token agent tree at 32,768 tokens per
    fragment the library and the oracle agree on it."""
    rng = np.random.default_rng([1002, 0])
    topo = agent_tree(rng)
    frags, info = b.fragment(topo.parent, topo.seg_start, topo.seg_len, 32768)
    ref = oracle.fragment(topo.parent, topo.seg_start, topo.seg_len, 32768)
    assert info["fragment_tokens"] == sum(len(r["source"]) for r in ref)
    assert info["source_tokens"] == topo.total_tokens
    assert all(len(f["source"]) <= 32768 for f in frags)
