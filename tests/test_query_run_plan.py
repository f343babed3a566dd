"""Query-run plans on the host (no GPU): the tile lists and pair counts a
run plan derives, checked against the oracle's visibility definition.

A run [q_begin, q_end) is one context-parallel rank's local queries (issue
"Shared-prefix training with context parallelism for exact agent
trajectories", section "Describe the solution you'd like"): its plan keeps
every key but only the run's queries.
"""

import ctypes

import numpy as np
import pytest

import oracle
import shared_prefix_tree_amd.binding as b
from workloads import random_forest


def host_run_plan(topo, qb, qe):
    return b.Plan(topo.parent, topo.seg_start, topo.seg_len, device=False, query_run=(qb, qe))


@pytest.mark.parametrize("seed", [41, 42, 43])
def test_run_pairs_and_query_tiles_follow_the_visible_sets(seed):
    rng = np.random.default_rng(seed)
    topo = random_forest(rng, max_tokens=300, max_len=80, max_depth=4, p_new_root=0.2)
    T = topo.total_tokens
    cuts = np.sort(rng.choice(np.arange(1, T), size=3, replace=False))
    edges = [0, *cuts.tolist(), T]
    total = 0
    st = np.asarray(topo.seg_start)
    for qb, qe in zip(edges[:-1], edges[1:]):
        p = host_run_plan(topo, qb, qe)
        info = p.info()
        assert (info["q_begin"], info["q_end"], info["total_tokens"]) == (qb, qe, T)
        want = sum(len(oracle.visible_tokens(topo, i)) for i in range(qb, qe))
        assert info["pairs"] == want
        total += info["pairs"]
        # 32-token query tiles: exactly the run's tokens, once each, never
        # crossing a segment, pos0 = the token's offset in its sequence
        tiles = p.export(b.EXPORT_Q_TILES)
        covered = np.zeros(T, int)
        for q0, nq, seg, pos0 in tiles:
            assert 1 <= nq <= 32
            assert st[seg] <= q0 and q0 + nq <= st[seg] + topo.seg_len[seg]
            assert pos0 == oracle.position_in_sequence(topo, q0)
            covered[q0:q0 + nq] += 1
        assert np.array_equal(covered[qb:qe], np.ones(qe - qb, int))
        assert not covered[:qb].any() and not covered[qe:].any()
        # key tiles: every key, with the subtree end of its segment
        kt = p.export(b.EXPORT_KV_TILES)
        keys = np.zeros(T, int)
        end = oracle.subtree_end(topo)
        for k0, nk, seg, qend in kt:
            keys[k0:k0 + nk] += 1
            assert qend == end[seg]
        assert np.array_equal(keys, np.ones(T, int))
        p.close()
    assert total == oracle.pairs(topo)


def test_run_validation():
    topo_args = ([-1, 0], [0, 10], [10, 5])
    lib = b.library()
    h = ctypes.c_void_p()
    for qb, qe in ((0, 0), (5, 3), (-1, 4), (0, 16), (15, 16)):
        p, pp = b._i32(topo_args[0])
        s, sp = b._i32(topo_args[1])
        n, np_ = b._i32(topo_args[2])
        rc = lib.tree_attn_plan_query_run_host(pp, sp, np_, 2, qb, qe, ctypes.byref(h))
        assert rc == b.INVALID_ARGUMENT, (qb, qe)
        assert "query run" in lib.tree_attn_last_error().decode()
    p = b.Plan(*topo_args, device=False, query_run=(0, 15))
    assert p.info()["pairs"] == oracle.pairs(
        __import__("workloads").Topology(*topo_args))


def test_run_partial_gradients_sum_to_the_whole_in_the_oracle():
    """The loss splits over the runs, so the oracle's dk / dv with dout zeroed
    outside each run sum (in float64, up to rounding) to the whole gradient,
    and its out / dq rows do not depend on the run."""
    rng = np.random.default_rng(44)
    topo = random_forest(rng, max_tokens=90, max_len=20, max_depth=3, p_new_root=0.2)
    T = topo.total_tokens
    q, k, v, do = (rng.standard_normal((T, h, 16)) for h in (2, 1, 1, 2))
    dq, dk, dv = oracle.backward(q, k, v, do, topo)
    edges = [0, T // 3, (2 * T) // 3, T]
    sdk, sdv = np.zeros_like(dk), np.zeros_like(dv)
    for qb, qe in zip(edges[:-1], edges[1:]):
        d = np.zeros_like(do)
        d[qb:qe] = do[qb:qe]
        dq_r, dk_r, dv_r = oracle.backward(q, k, v, d, topo)
        np.testing.assert_allclose(dq_r[qb:qe], dq[qb:qe], rtol=1e-12, atol=1e-12)
        sdk += dk_r
        sdv += dv_r
    np.testing.assert_allclose(sdk, dk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sdv, dv, rtol=1e-10, atol=1e-12)
