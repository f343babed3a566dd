"""GPU: Mamba state forking (tree-causal convolution and state-space
recurrence) against the float64 oracle.

Draft "feat(hybrid): add opt-in shared-prefix attention and Mamba
execution" (intro): the recurrent state forks into each branch, the
convolution halo runs per branch, and backward accumulates the branches into
the shared prefix.  Everything is float32; the bound is the float32 one of
the attention path (rel-L2 1e-5; the pages' own float32 tree comparisons of
the Mamba path were within about 1.2e-5).  Two runs are bitwise equal.
"""

import numpy as np
import pytest

import oracle
from tests.parity_util import log, rel_l2
from workloads import mamba_tensors, random_forest, tiny_tree

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-5


def dev_tensors(d, dev):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items()}


def forests():
    rng = np.random.default_rng(61)
    return {
        "tiny_tree": tiny_tree(),
        "forest_long_segments": random_forest(rng, max_tokens=900, max_len=300, max_depth=4, p_new_root=0.1),
        "forest_short_segments": random_forest(rng, max_tokens=500, max_len=20, max_depth=6, p_new_root=0.1),
    }


@pytest.mark.parametrize("name", ["tiny_tree", "forest_long_segments", "forest_short_segments"])
@pytest.mark.parametrize("width", [4, 3, 1])
def test_conv_matches_oracle(name, width):
    import shared_prefix_tree_amd as sp

    topo = forests()[name]
    T = topo.total_tokens
    d = mamba_tensors(70 + width, T, channels=96, width=width)
    rng = np.random.default_rng(width)
    dy = rng.standard_normal((T, 96)).astype(np.float32)
    dev = "cuda:0"
    t = dev_tensors({"x": d["conv_x"], "w": d["conv_w"], "b": d["conv_b"], "dy": dy}, dev)
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    y = sp.conv_fwd(t["x"], t["w"], t["b"], plan)
    dx, dw, db = sp.conv_bwd(t["x"], t["w"], t["dy"], plan)
    torch.cuda.synchronize()
    y_ref = oracle.conv_forward(d["conv_x"], d["conv_w"], d["conv_b"], topo)
    dx_ref, dw_ref, db_ref = oracle.conv_backward(dy, d["conv_x"], d["conv_w"], topo)
    errs = {k: rel_l2(g.cpu().numpy(), r) for k, g, r in
            (("y", y, y_ref), ("dx", dx, dx_ref), ("dw", dw, dw_ref), ("db", db, db_ref))}
    log(f"conv {name} T={T} width={width}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs
    y2 = sp.conv_fwd(t["x"], t["w"], t["b"], plan)
    g2 = sp.conv_bwd(t["x"], t["w"], t["dy"], plan)
    assert torch.equal(y, y2) and all(torch.equal(a, b) for a, b in zip((dx, dw, db), g2))


@pytest.mark.parametrize("name", ["tiny_tree", "forest_long_segments", "forest_short_segments"])
@pytest.mark.parametrize("N,H,G", [(128, 4, 2), (64, 6, 3)])
def test_ssm_forward_matches_oracle(name, N, H, G):
    import shared_prefix_tree_amd as sp

    topo = forests()[name]
    T = topo.total_tokens
    d = mamba_tensors(80 + N, T, heads=H, groups=G, state_dim=N)
    dev = "cuda:0"
    keys = ("x", "dt", "A", "B", "C", "D")
    t = dev_tensors({k: d[k] for k in keys}, dev)
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    log(f"ssm fwd {name}: T={T} units={plan.info()['num_units']} H={H} G={G} N={N}")
    y, states = sp.ssm_fwd(*(t[k] for k in keys), plan)
    torch.cuda.synchronize()
    y_ref = oracle.ssm_forward(*(d[k] for k in keys), topo)
    e = rel_l2(y.cpu().numpy(), y_ref)
    # the saved state before each 32-token chunk of a unit is the oracle's
    # state after the chunk's predecessor token
    S_ref = oracle.ssm_states(d["x"], d["dt"], d["A"], d["B"], topo)
    st, ln = plan.export("unit_start"), plan.export("unit_len")
    prev = oracle.previous_token(topo)
    cpu = plan.info()["unit_tokens"] // 32
    saved = states[: st.size * cpu * H * 64 * N * 4].view(torch.float32).view(st.size, cpu, H, 64, N).cpu().numpy()
    got, ref = [], []
    for u in range(st.size):
        for c in range(-(-int(ln[u]) // 32)):
            first = int(st[u]) + 32 * c
            got.append(saved[u, c])
            ref.append(S_ref[prev[first]] if prev[first] >= 0 else np.zeros_like(S_ref[0]))
    got, ref = np.stack(got), np.stack(ref)
    e_s = rel_l2(got, ref) if np.any(ref) else float(np.abs(got).max())
    log(f"  y rel-L2 {e:.2e}, saved states rel-L2 {e_s:.2e}")
    assert e <= TOL and e_s <= TOL
    y2, _ = sp.ssm_fwd(*(t[k] for k in keys), plan)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("name", ["tiny_tree", "forest_long_segments", "forest_short_segments"])
@pytest.mark.parametrize("N,H,G", [(128, 4, 2), (64, 6, 3), (64, 3, 1), (64, 8, 1)])
def test_ssm_backward_matches_oracle(name, N, H, G):
    """Every gradient against the oracle; a branch point's state gets the sum
    of its branches (the forests have forks inside and at the end of units).
    The shapes give the gradient pass 2, 2, 1 and 4 heads per block (the
    largest of 4, 2, 1 that divides the heads of a group)."""
    import shared_prefix_tree_amd as sp

    topo = forests()[name]
    T = topo.total_tokens
    d = mamba_tensors(90 + N, T, heads=H, groups=G, state_dim=N)
    dy = np.random.default_rng(N + H).standard_normal((T, H, 64)).astype(np.float32)
    dev = "cuda:0"
    keys = ("x", "dt", "A", "B", "C", "D")
    t = dev_tensors({k: d[k] for k in keys}, dev)
    dyt = torch.from_numpy(dy).to(dev)
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    log(f"ssm bwd {name}: T={T} units={plan.info()['num_units']} H={H} G={G} N={N}")
    _, states = sp.ssm_fwd(*(t[k] for k in keys), plan)
    got = sp.ssm_bwd(*(t[k] for k in keys), dyt, plan, states)
    torch.cuda.synchronize()
    ref = oracle.ssm_backward(dy, *(d[k] for k in keys), topo)
    errs = {}
    for k, g, r in zip(("dx", "ddt", "dA", "dB", "dC", "dD"), got, ref):
        errs[k] = rel_l2(g.cpu().numpy(), r)
    log("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs
    again = sp.ssm_bwd(*(t[k] for k in keys), dyt, plan, states)
    assert all(torch.equal(a, b) for a, b in zip(got, again))


def test_ssm_rejects_unsupported_shapes():
    import shared_prefix_tree_amd as sp

    dev = "cuda:0"
    topo = tiny_tree()
    T = topo.total_tokens
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    z = lambda *s: torch.zeros(*s, dtype=torch.float32, device=dev)  # noqa: E731
    with pytest.raises(sp.TreeAttnError, match="head_dim must be 64"):
        sp.ssm_fwd(z(T, 2, 32), z(T, 2), z(2), z(T, 1, 64), z(T, 1, 64), z(2), plan)
    with pytest.raises(sp.TreeAttnError, match="state_dim"):
        sp.ssm_fwd(z(T, 2, 64), z(T, 2), z(2), z(T, 1, 32), z(T, 1, 32), z(2), plan)
    with pytest.raises(sp.TreeAttnError, match="multiple of 4"):
        sp.conv_fwd(z(T, 6), z(6, 4), z(6), plan)


def test_token_count_must_match_the_plan():
    """A tensor with fewer or more rows than the plan is rejected before any
    launch: by the binding (ValueError) and by the C ABI (INVALID_ARGUMENT,
    outputs untouched)."""
    import ctypes

    import shared_prefix_tree_amd as sp
    from shared_prefix_tree_amd import binding as b

    dev = "cuda:0"
    topo = tiny_tree()
    T = topo.total_tokens
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    assert plan.num_tokens == T
    z = lambda *s: torch.zeros(*s, dtype=torch.float32, device=dev)  # noqa: E731
    for rows in (T - 1, T + 5):
        with pytest.raises(ValueError, match="rows"):
            sp.conv_fwd(z(rows, 8), z(8, 4), z(8), plan)
        with pytest.raises(ValueError, match="rows"):
            sp.conv_bwd(z(rows, 8), z(8, 4), z(rows, 8), plan)
        with pytest.raises(ValueError, match="rows"):
            sp.ssm_fwd(z(rows, 2, 64), z(rows, 2), z(2), z(rows, 1, 64), z(rows, 1, 64), z(2), plan)
        with pytest.raises(ValueError, match="rows"):
            sp.ssm_bwd(z(rows, 2, 64), z(rows, 2), z(2), z(rows, 1, 64), z(rows, 1, 64), z(2), z(rows, 2, 64),
                       plan, z(64))
    lib = sp.library()
    x, w, bias = z(T, 8), z(8, 4), z(8)
    y = torch.full((T, 8), 7.0, device=dev)
    ws = torch.zeros(max(256, lib.tree_attn_conv_bwd_workspace_bytes(plan.handle, 8, 4)), dtype=torch.uint8,
                     device=dev)
    dx, dw, db = torch.full((T, 8), 7.0, device=dev), torch.full((8, 4), 7.0, device=dev), torch.full((8,), 7.0, device=dev)
    for rows in (T - 1, T + 1, 0):
        assert lib.tree_attn_conv_fwd(x.data_ptr(), w.data_ptr(), bias.data_ptr(), rows, 8, 4, plan.handle,
                                      y.data_ptr(), None) == b.INVALID_ARGUMENT
        assert "num_tokens" in lib.tree_attn_last_error().decode()
        assert lib.tree_attn_conv_bwd(x.data_ptr(), w.data_ptr(), x.data_ptr(), rows, 8, 4, plan.handle,
                                      dx.data_ptr(), dw.data_ptr(), db.data_ptr(), ws.data_ptr(), ws.numel(),
                                      None) == b.INVALID_ARGUMENT
    H, P, G, N = 2, 64, 1, 64
    xs, dts, As, Bs, Ds = z(T, H, P), z(T, H), z(H), z(T, G, N), z(H)
    ys = torch.full((T, H, P), 7.0, device=dev)
    good = b.SsmShape(T, H, P, G, N)
    st = torch.zeros(max(256, lib.tree_attn_ssm_states_bytes(plan.handle, ctypes.byref(good))), dtype=torch.uint8,
                     device=dev)
    wsf = torch.zeros(max(256, lib.tree_attn_ssm_workspace_bytes(plan.handle, ctypes.byref(good))),
                      dtype=torch.uint8, device=dev)
    for rows in (T - 1, T + 1):
        bad = b.SsmShape(rows, H, P, G, N)
        assert lib.tree_attn_ssm_fwd(xs.data_ptr(), dts.data_ptr(), As.data_ptr(), Bs.data_ptr(), Bs.data_ptr(),
                                     Ds.data_ptr(), plan.handle, ctypes.byref(bad), ys.data_ptr(), st.data_ptr(),
                                     st.numel(), wsf.data_ptr(), wsf.numel(), None) == b.INVALID_ARGUMENT
        assert "num_tokens" in lib.tree_attn_last_error().decode()
    torch.cuda.synchronize()
    for t in (y, dx, dw, db, ys):
        assert torch.all(t == 7.0)


def test_ssm_at_the_benchmark_shape_on_two_groups():
    """The benchmark's mixer shape (128 heads x 64, 8 groups, state 128) on a
    ~1,000-token forest.  A group's heads read only that group's B and C, so
    the oracle run on the 16 heads of one group alone gives exactly those
    heads' outputs and the group's dB / dC; groups 0 and 7 are checked."""
    import shared_prefix_tree_amd as sp

    H, G, N = 128, 8, 128
    rng = np.random.default_rng(97)
    topo = random_forest(rng, max_tokens=1100, max_len=260, max_depth=5, p_new_root=0.05)
    T = topo.total_tokens
    d = mamba_tensors(97, T, heads=H, groups=G, state_dim=N)
    dy = rng.standard_normal((T, H, 64)).astype(np.float32)
    dev = "cuda:0"
    keys = ("x", "dt", "A", "B", "C", "D")
    t = dev_tensors({k: d[k] for k in keys}, dev)
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    log(f"ssm benchmark shape: T={T} units={plan.info()['num_units']}")
    y, states = sp.ssm_fwd(*(t[k] for k in keys), plan)
    grads = sp.ssm_bwd(*(t[k] for k in keys), torch.from_numpy(dy).to(dev), plan, states)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    dx, ddt, dA, dB, dC, dD = (g.cpu().numpy() for g in grads)
    hpg = H // G
    for g in (0, G - 1):
        hs = slice(g * hpg, (g + 1) * hpg)
        sub = {"x": d["x"][:, hs], "dt": d["dt"][:, hs], "A": d["A"][hs], "B": d["B"][:, g:g + 1],
               "C": d["C"][:, g:g + 1], "D": d["D"][hs]}
        y_ref = oracle.ssm_forward(*(sub[k] for k in keys), topo)
        ref = oracle.ssm_backward(dy[:, hs], *(sub[k] for k in keys), topo)
        got = (dx[:, hs], ddt[:, hs], dA[hs], dB[:, g:g + 1], dC[:, g:g + 1], dD[hs])
        errs = {"y": rel_l2(y[:, hs], y_ref)}
        errs.update({k: rel_l2(a, r) for k, a, r in zip(("dx", "ddt", "dA", "dB", "dC", "dD"), got, ref)})
        log(f"  group {g}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
        assert all(v <= TOL for v in errs.values()), (g, errs)


def edge_forests():
    from workloads import Topology

    def dfs(nodes):
        parent = np.array([p for p, _ in nodes])
        ln = np.array([n for _, n in nodes])
        st = np.concatenate([[0], np.cumsum(ln)[:-1]])
        return Topology(parent, st, ln)

    return {
        "one_token": dfs([(-1, 1)]),
        "one_unit": dfs([(-1, 128)]),
        "unit_plus_one": dfs([(-1, 129)]),
        "fork_at_unit_end": dfs([(-1, 128), (0, 1), (0, 33), (0, 128)]),
        "chain_of_single_tokens": dfs([(-1, 1), (0, 1), (1, 1), (2, 1), (3, 1), (4, 1), (4, 2)]),
        "two_roots": dfs([(-1, 40), (0, 3), (-1, 200), (2, 64)]),
    }


@pytest.mark.parametrize("name", list(edge_forests()))
def test_mamba_edge_topologies(name):
    """Degenerate forests: one token, exactly one unit and one past it, a
    fork right at a unit end, chains of one-token segments, several roots."""
    import shared_prefix_tree_amd as sp

    topo = edge_forests()[name]
    T = topo.total_tokens
    H, G, N = 4, 2, 64
    d = mamba_tensors(131, T, heads=H, groups=G, state_dim=N, channels=8, width=4)
    rng = np.random.default_rng(132)
    dy = rng.standard_normal((T, H, 64)).astype(np.float32)
    dcy = rng.standard_normal((T, 8)).astype(np.float32)
    dev = "cuda:0"
    keys = ("x", "dt", "A", "B", "C", "D")
    t = dev_tensors({k: d[k] for k in keys}, dev)
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    y, states = sp.ssm_fwd(*(t[k] for k in keys), plan)
    got = sp.ssm_bwd(*(t[k] for k in keys), torch.from_numpy(dy).to(dev), plan, states)
    c = dev_tensors({"x": d["conv_x"], "w": d["conv_w"], "b": d["conv_b"], "dy": dcy}, dev)
    cy = sp.conv_fwd(c["x"], c["w"], c["b"], plan)
    cg = sp.conv_bwd(c["x"], c["w"], c["dy"], plan)
    torch.cuda.synchronize()
    ref = {"y": oracle.ssm_forward(*(d[k] for k in keys), topo)}
    ref.update(zip(("dx", "ddt", "dA", "dB", "dC", "dD"), oracle.ssm_backward(dy, *(d[k] for k in keys), topo)))
    ref["cy"] = oracle.conv_forward(d["conv_x"], d["conv_w"], d["conv_b"], topo)
    ref.update(zip(("cdx", "cdw", "cdb"), oracle.conv_backward(dcy, d["conv_x"], d["conv_w"], topo)))
    gots = {"y": y, **dict(zip(("dx", "ddt", "dA", "dB", "dC", "dD"), got)), "cy": cy,
            **dict(zip(("cdx", "cdw", "cdb"), cg))}
    errs = {k: rel_l2(gots[k].cpu().numpy(), ref[k]) for k in ref}
    log(f"mamba edge {name} T={T}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs
