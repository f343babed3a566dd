"""GPU: the allocation-free backward (``tree_attn_bwd_noalloc``, workspace in
the library's fixed device scratch) against ``tree_attn_bwd`` with a caller
workspace, through the C ABI: bitwise equal on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents),
and shapes above the scratch limit rejected before any launch."""

import ctypes

import numpy as np
import pytest

from tests.parity_util import log, to_torch
from workloads import f32_to_bf16, random_forest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _inputs(rng, topo, Hq, Hkv, D):
    arrs = {n: f32_to_bf16(rng.standard_normal((topo.total_tokens, h, D)).astype(np.float32))
            for n, h in (("q", Hq), ("k", Hkv), ("v", Hkv), ("dout", Hq))}
    return {n: to_torch(a, "bf16", "cuda:0") for n, a in arrs.items()}


def test_noalloc_backward_matches_the_workspace_backward():
    import shared_prefix_tree_amd as sp
    from shared_prefix_tree_amd import binding as b

    lib = sp.library()
    rng = np.random.default_rng(77)
    cases = [
        (random_forest(rng, max_tokens=3000, max_len=600, max_depth=5, p_new_root=0.05), 16, 4),
        (random_forest(rng, max_tokens=700, max_len=150, max_depth=4), 8, 2),  # smaller second call
    ]
    for n, (topo, Hq, Hkv) in enumerate(cases):
        log(f"noalloc call {n}: T={topo.total_tokens} S={topo.num_segments} Hq={Hq} Hkv={Hkv} D=128 bf16")
        t = _inputs(rng, topo, Hq, Hkv, 128)
        plan = sp.Plan.from_topology(topo)
        out, lse = sp.tree_attn_fwd(t["q"], t["k"], t["v"], plan)
        ref = sp.tree_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], plan)
        got = [torch.full_like(x, 7.0) for x in ref]
        shape = b._shape(t["q"], t["k"], 0.0)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.tree_attn_bwd_noalloc(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), t["dout"].data_ptr(), plan.handle, ctypes.byref(shape),
                                       got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), stream)
        assert rc == b.OK, lib.tree_attn_last_error().decode()
        torch.cuda.synchronize()
        for name, a, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, g), (n, name)
        # the binding wrapper gives the same
        again = sp.tree_attn_bwd_noalloc(t["q"], t["k"], t["v"], out, lse, t["dout"], plan,
                                         *(torch.empty_like(x) for x in ref))
        torch.cuda.synchronize()
        for a, g in zip(ref, again):
            assert torch.equal(a, g)


def test_noalloc_rejects_shapes_above_the_scratch_limit():
    import shared_prefix_tree_amd as sp
    from shared_prefix_tree_amd import binding as b

    lib = sp.library()
    # a single segment of 262,145 tokens with 32 query heads: Hq * T > 2^23
    T = (1 << 18) + 1
    plan = sp.Plan(np.array([-1]), np.array([0]), np.array([T]))
    shape = b.Shape(T, 32, 8, 128, b.BF16, 0.0)
    dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda:0")
    p = dummy.data_ptr()
    rc = lib.tree_attn_bwd_noalloc(p, p, p, p, p, p, plan.handle, ctypes.byref(shape), p, p, p, None)
    assert rc == b.UNSUPPORTED
    assert "scratch" in lib.tree_attn_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(dummy == 0)
