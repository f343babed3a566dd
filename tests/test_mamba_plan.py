"""Host tables of the Mamba plan (no GPU): each token's predecessor against
the oracle's definition, and the scan units (cover every segment in order,
never cross a segment, predecessor = previous unit or the parent's last)."""

import numpy as np
import pytest

import oracle
import shared_prefix_tree_amd as sp
from shared_prefix_tree_amd import binding as b
from workloads import WORKLOADS, random_forest, tiny_tree


def topologies():
    rng = np.random.default_rng(11)
    out = [tiny_tree()] + [random_forest(rng, max_tokens=3000, max_len=400, max_depth=5) for _ in range(6)]
    out += [w.topology() for w in WORKLOADS[:3]]
    return out


@pytest.mark.parametrize("idx", range(10))
def test_mamba_plan_tables(idx):
    topo = topologies()[idx]
    plan = sp.MambaPlan.from_topology(topo, device=False)
    info = plan.info()
    assert info["num_tokens"] == topo.total_tokens and info["num_segments"] == topo.num_segments
    assert np.array_equal(plan.export("prev"), oracle.previous_token(topo))
    st, ln, pr = plan.export("unit_start"), plan.export("unit_len"), plan.export("unit_pred")
    L = info["unit_tokens"]
    assert st.size == info["num_units"] == ln.size == pr.size
    assert np.all((ln >= 1) & (ln <= L))
    assert st[0] == 0 and np.all(st[1:] == st[:-1] + ln[:-1])  # contiguous, DFS order
    seg_of = np.repeat(np.arange(topo.num_segments), topo.seg_len)
    last_unit = {}
    for u in range(st.size):
        s = seg_of[st[u]]
        assert seg_of[st[u] + ln[u] - 1] == s  # never crosses a segment
        if st[u] == topo.seg_start[s]:
            p = topo.parent[s]
            assert pr[u] == (-1 if p < 0 else last_unit[p])
        else:
            assert pr[u] == u - 1 and ln[u - 1] == L
        last_unit[s] = u


def test_mamba_plan_rejects_malformed_forests():
    with pytest.raises(b.TreeAttnError, match="tree_attn_mamba_plan_host"):
        sp.MambaPlan([-1, 1], [0, 4], [4, 4], device=False)  # parent not earlier
    with pytest.raises(b.TreeAttnError):
        sp.MambaPlan([-1, 0], [0, 5], [4, 4], device=False)  # not contiguous
