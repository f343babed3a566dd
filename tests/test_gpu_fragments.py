"""GPU: attention over bounded fragments with repeated ancestors is exact.

Issue "Shared-prefix training with context parallelism for exact agent
trajectories" (section "Describe the solution you'd like") bounds fragments
and repeats ancestors across them.  Running the library on each fragment of
``tree_attn_fragment`` -- rows gathered from the source tensors, dout zero on
repeated (non-owned) rows -- must reproduce the unfragmented run: out, lse
and dq of every owned token bitwise (its key sequence is the same, in the
same order), and dk / dv once the fragments' rows are summed back onto their
source tokens (each copy receives the gradient of the owned queries of its
fragment), against the whole run and against the float64 oracle.
"""

import numpy as np
import pytest

import oracle
from tests.parity_util import log, oracle_inputs, rel_l2, tensor_error, to_host, to_torch
from workloads import Topology, f32_to_bf16, random_forest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D,Hq,Hkv,seed", [("bf16", 128, 8, 2, 71), ("fp32", 64, 4, 2, 72),
                                                 ("bf16", 64, 4, 1, 73)])
def test_fragments_reproduce_the_whole_forest(dtype, D, Hq, Hkv, seed):
    import shared_prefix_tree_amd as sp

    rng = np.random.default_rng(seed)
    topo = random_forest(rng, max_tokens=800, max_len=120, max_depth=5, p_new_root=0.1)
    T = topo.total_tokens
    longest = max(len(oracle.visible_tokens(topo, i)) for i in range(T))
    bound = longest + 37
    arrs = {}
    for name, h in (("q", Hq), ("k", Hkv), ("v", Hkv), ("dout", Hq)):
        x = rng.standard_normal((T, h, D)).astype(np.float32)
        arrs[name] = f32_to_bf16(x) if dtype == "bf16" else x
    dev = "cuda:0"
    t = {k: to_torch(v, dtype, dev) for k, v in arrs.items()}
    with torch.cuda.device(dev):
        whole = sp.Plan.from_topology(topo)
    out, lse = sp.tree_attn_fwd(t["q"], t["k"], t["v"], whole)
    dq, dk, dv = sp.tree_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], whole)

    frags, info = sp.fragment(topo.parent, topo.seg_start, topo.seg_len, bound)
    log(f"fragments {dtype}: T={T} bound={bound} fragments={info['num_fragments']} "
        f"tokens {info['fragment_tokens']} (+{info['fragment_tokens'] / T - 1:.1%})")
    assert info["num_fragments"] >= 2
    sum_dk = torch.zeros(dk.shape, dtype=torch.float64, device=dev)
    sum_dv = torch.zeros_like(sum_dk)
    for fr in frags:
        src = torch.from_numpy(fr["source"].astype(np.int64)).to(dev)
        own = torch.from_numpy(fr["owner"].astype(bool)).to(dev)
        sub = Topology(fr["parent"].tolist(), fr["seg_start"].tolist(), fr["seg_len"].tolist())
        with torch.cuda.device(dev):
            plan = sp.Plan.from_topology(sub)
        fq, fk, fv = t["q"][src].contiguous(), t["k"][src].contiguous(), t["v"][src].contiguous()
        fdo = t["dout"][src].clone()
        fdo[~own] = 0
        fo, fl = sp.tree_attn_fwd(fq, fk, fv, plan)
        fdq, fdk, fdv = sp.tree_attn_bwd(fq, fk, fv, fo, fl, fdo, plan)
        torch.cuda.synchronize()
        rows = src[own]
        assert torch.equal(fo[own], out[rows])
        assert torch.equal(fl[:, own], lse[:, rows])
        assert torch.equal(fdq[own], dq[rows])
        sum_dk.index_add_(0, src, fdk.double())
        sum_dv.index_add_(0, src, fdv.double())
    x = oracle_inputs(arrs, dtype)
    _, dk_ref, dv_ref = oracle.backward(x["q"], x["k"], x["v"], x["dout"], topo)
    for name, s, whole_g, ref in (("dk", sum_dk, dk, dk_ref), ("dv", sum_dv, dv, dv_ref)):
        e_whole = rel_l2(s.cpu().numpy(), to_host(whole_g))
        err, bound_ = tensor_error(name, s.cpu().numpy(), ref, dtype)
        log(f"  {name}: summed over copies vs whole run rel-L2 {e_whole:.3%}; vs oracle {err:.3g} (<= {bound_:.0e})")
        assert err <= bound_
        assert e_whole <= (2.5e-2 if dtype == "bf16" else 1e-5)
