"""GPU: query runs, one context-parallel rank's share of the path.

Issue "Shared-prefix training with context parallelism for exact agent
trajectories" (section "Describe the solution you'd like") keeps queries
local to their rank and gathers K/V: a rank computes attention for its own
tokens against every key.  A plan built by ``tree_attn_plan_query_run`` for
the tokens [q_begin, q_end) is that share.  Over a partition of [0, T) into
runs, each run

* writes out, lse and dq of its rows only, bitwise equal to the whole-token
  plan's rows (the page's validation reports CP2 outputs and Q gradients as
  exact) and leaves every other row untouched;
* writes all of dk and dv: the gradient of its part of the loss, which the
  float64 oracle gives by zeroing dout outside the run; the shares summed
  over the runs match the whole plan's dk / dv (the page's CP2 K/V gradients
  were within 0.4792 % rel-L2 of CP1 against a 2.5 % threshold).
"""

import numpy as np
import pytest

import oracle
from tests.parity_util import log, oracle_inputs, rel_l2, tensor_error, to_host, to_torch
from workloads import f32_to_bf16, random_forest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def make_inputs(rng, T, Hq, Hkv, D, dtype):
    arrs = {}
    for name, h in (("q", Hq), ("k", Hkv), ("v", Hkv), ("dout", Hq)):
        x = rng.standard_normal((T, h, D)).astype(np.float32)
        arrs[name] = f32_to_bf16(x) if dtype == "bf16" else x
    return arrs


def partition(rng, T, R):
    cuts = np.sort(rng.choice(np.arange(1, T), size=R - 1, replace=False))
    edges = [0, *cuts.tolist(), T]
    return list(zip(edges[:-1], edges[1:]))


CASES = [
    # (label, dtype, head_dim, Hq, Hkv, ranks, seed)
    ("bf16_r3", "bf16", 128, 8, 2, 3, 21),
    ("bf16_d64_r4", "bf16", 64, 8, 2, 4, 22),
    ("fp32_r2", "fp32", 64, 4, 2, 2, 23),
    ("bf16_r5_g1", "bf16", 128, 2, 2, 5, 24),
]


@pytest.mark.parametrize("label,dtype,D,Hq,Hkv,R,seed", CASES, ids=[c[0] for c in CASES])
def test_query_runs_partition_the_whole_plan(label, dtype, D, Hq, Hkv, R, seed):
    import shared_prefix_tree_amd as sp

    rng = np.random.default_rng(seed)
    topo = random_forest(rng, max_tokens=600, max_len=150, max_depth=5, p_new_root=0.1)
    T = topo.total_tokens
    arrs = make_inputs(rng, T, Hq, Hkv, D, dtype)
    runs = partition(rng, T, R)
    log(f"query runs {label}: T={T} S={topo.num_segments} runs={runs}")
    dev = "cuda:0"
    t = {k: to_torch(v, dtype, dev) for k, v in arrs.items()}
    with torch.cuda.device(dev):
        whole = sp.Plan.from_topology(topo)
    out, lse = sp.tree_attn_fwd(t["q"], t["k"], t["v"], whole)
    dq, dk, dv = sp.tree_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], whole)

    x = oracle_inputs(arrs, dtype)
    sum_dk = torch.zeros(dk.shape, dtype=torch.float64, device=dev)
    sum_dv = torch.zeros_like(sum_dk)
    pairs = 0
    for qb, qe in runs:
        with torch.cuda.device(dev):
            plan = sp.Plan.from_topology(topo, query_run=(qb, qe))
        info = plan.info()
        assert (info["q_begin"], info["q_end"]) == (qb, qe)
        pairs += info["pairs"]
        out_r = torch.full_like(out, SENTINEL)
        lse_r = torch.full_like(lse, SENTINEL)
        dq_r = torch.full_like(dq, SENTINEL)
        dk_r = torch.full_like(dk, SENTINEL)
        dv_r = torch.full_like(dv, SENTINEL)
        sp.tree_attn_fwd(t["q"], t["k"], t["v"], plan, out=out_r, lse=lse_r)
        sp.tree_attn_bwd(t["q"], t["k"], t["v"], out_r, lse_r, t["dout"], plan, dq=dq_r, dk=dk_r, dv=dv_r)
        torch.cuda.synchronize()
        # other rows untouched; the run's rows bitwise those of the whole plan
        for name, got, ref, rows in (("out", out_r, out, slice(qb, qe)), ("dq", dq_r, dq, slice(qb, qe))):
            outside = torch.cat([got[:qb], got[qe:]])
            assert bool((outside == SENTINEL).all()), (label, name, qb, qe)
            assert torch.equal(got[rows], ref[rows]), (label, name, qb, qe)
        outside = torch.cat([lse_r[:, :qb], lse_r[:, qe:]], dim=1)
        assert bool((outside == SENTINEL).all()), (label, "lse", qb, qe)
        assert torch.equal(lse_r[:, qb:qe], lse[:, qb:qe]), (label, "lse", qb, qe)
        # dk / dv: the run's share against the oracle with dout zeroed elsewhere
        dout_run = np.zeros_like(x["dout"])
        dout_run[qb:qe] = x["dout"][qb:qe]
        _, dk_ref, dv_ref = oracle.backward(x["q"], x["k"], x["v"], dout_run, topo)
        for name, got, ref in (("dk", dk_r, dk_ref), ("dv", dv_r, dv_ref)):
            err, bound = tensor_error(name, to_host(got), ref, dtype)
            log(f"  run [{qb}, {qe}) {name} share error {err:.3g} (<= {bound:.0e})")
            assert err <= bound, (label, name, qb, qe, err)
        sum_dk += dk_r.double()
        sum_dv += dv_r.double()
    assert pairs == whole.info()["pairs"]
    for name, s, ref in (("dk", sum_dk, dk), ("dv", sum_dv, dv)):
        e = rel_l2(s.cpu().numpy(), to_host(ref))
        log(f"  sum over runs vs whole plan: {name} rel-L2 {e:.4%}")
        assert e <= 2.5e-2 if dtype == "bf16" else e <= 1e-5, (label, name, e)


def test_query_run_of_one_token_in_a_leaf():
    """A run of a single leaf token: its row matches the whole plan, and keys
    outside its ancestor path get exactly zero gradients."""
    import shared_prefix_tree_amd as sp

    rng = np.random.default_rng(31)
    topo = random_forest(rng, max_tokens=400, max_len=120, max_depth=4, p_new_root=0.0)
    T = topo.total_tokens
    arrs = make_inputs(rng, T, 4, 2, 128, "bf16")
    dev = "cuda:0"
    t = {k: to_torch(v, "bf16", dev) for k, v in arrs.items()}
    i = T - 1  # the last token: the end of a leaf segment
    with torch.cuda.device(dev):
        whole = sp.Plan.from_topology(topo)
        plan = sp.Plan.from_topology(topo, query_run=(i, i + 1))
    log(f"one-token run: T={T} token {i}")
    out, lse = sp.tree_attn_fwd(t["q"], t["k"], t["v"], whole)
    dq, _, _ = sp.tree_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], whole)
    out_r = torch.full_like(out, SENTINEL)
    lse_r = torch.full_like(lse, SENTINEL)
    sp.tree_attn_fwd(t["q"], t["k"], t["v"], plan, out=out_r, lse=lse_r)
    dq_r, dk_r, dv_r = sp.tree_attn_bwd(t["q"], t["k"], t["v"], out_r, lse_r, t["dout"], plan)
    torch.cuda.synchronize()
    assert torch.equal(out_r[i], out[i]) and torch.equal(lse_r[:, i], lse[:, i]) and torch.equal(dq_r[i], dq[i])
    # keys the token does not see: exactly zero; the ones it sees: not all zero
    seen = np.zeros(T, bool)
    seen[oracle.visible_tokens(topo, i)] = True
    for g in (dk_r, dv_r):
        h = to_host(g)
        assert np.all(h[~seen] == 0.0)
        assert np.any(h[seen] != 0.0)


def test_query_runs_before_and_inside_descendants():
    """Runs whose ends cut the 128-key dK/dV walk's two query ranges (a
    segment's descendants, then its own queries) in the degenerate ways: a run
    that ends hundreds of tokens before most key tiles (no query of the run
    sees them: exactly zero gradients), and runs that lie only among a
    segment's descendants or only in its own queries.  dk / dv against the
    float64 oracle with dout zeroed outside the run."""
    import shared_prefix_tree_amd as sp
    from workloads import long_chain

    rng = np.random.default_rng(5)
    # trunk segments 0, 1, 3, 4 with side leaves 2 and 5 (1,400 tokens)
    topo = long_chain(rng, total=1400, trunk=4, every=2, side_lo=100, side_hi=200)
    T = topo.total_tokens
    arrs = make_inputs(rng, T, 8, 2, 128, "bf16")
    dev = "cuda:0"
    t = {k: to_torch(v, "bf16", dev) for k, v in arrs.items()}
    x = oracle_inputs(arrs, "bf16")
    for qb, qe in ((0, 100), (600, 700), (1000, 1010), (270, 530)):
        with torch.cuda.device(dev):
            plan = sp.Plan.from_topology(topo, query_run=(qb, qe))
        log(f"run [{qb}, {qe}) of T={T}")
        out, lse = sp.tree_attn_fwd(t["q"], t["k"], t["v"], plan)
        _, dk, dv = sp.tree_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], plan)
        torch.cuda.synchronize()
        dout_run = np.zeros_like(x["dout"])
        dout_run[qb:qe] = x["dout"][qb:qe]
        _, dk_ref, dv_ref = oracle.backward(x["q"], x["k"], x["v"], dout_run, topo)
        seen = np.zeros(T, bool)
        for i in range(qb, qe):
            seen[oracle.visible_tokens(topo, i)] = True
        for name, got, ref in (("dk", dk, dk_ref), ("dv", dv, dv_ref)):
            h = to_host(got)
            err, bound = tensor_error(name, h, ref, "bf16")
            log(f"  {name} error {err:.3g} (<= {bound:.0e}); unseen keys {int((~seen).sum())}")
            assert err <= bound, (qb, qe, name, err)
            assert np.all(h[~seen] == 0.0), (qb, qe, name)
