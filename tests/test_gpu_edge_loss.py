"""GPU: sampled-edge projection and loss against the float64 oracle.

Only the hidden states that are the source of a sampled edge go through the
vocabulary head, each sampled action owning its loss once (Megatron-LM pull
request 7387, section "Summary"; issue "Shared-prefix training with context
parallelism for exact agent trajectories", section "Describe the solution
you'd like").

Bounds: inputs are bf16, logits and row statistics fp32, so loss and lse
are held to the lse bound of the attention path for bf16 inputs (max-abs
1e-3); dh and dW are bf16 results of bf16-rounded G, held to the gradient
bound (rel-L2 2.5e-2).  Tokens that are no edge's source get exactly zero
rows.  Two runs are bitwise equal (no atomics anywhere).
"""

import numpy as np
import pytest

import oracle
from tests.parity_util import log, rel_l2, to_host
from workloads import bf16_to_f32, make_tensor, random_forest, sampled_edges

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOSS_TOL = 1e-3
GRAD_TOL = 2.5e-2


def bf16_tensor(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def make_case(seed, T_max, d, V, p_sampled, w_std):
    rng = np.random.default_rng(seed)
    topo = random_forest(rng, max_tokens=T_max, max_len=max(8, T_max // 6), max_depth=5, p_new_root=0.1)
    src, tgt = sampled_edges(topo, rng, V, p_sampled)
    if src.size == 0:  # at least one edge
        src, tgt = np.array([0], np.int32), np.array([V - 1], np.int32)
    T = topo.total_tokens
    h = make_tensor("hidden", seed, T, 1, d)[:, 0]
    w = make_tensor("weight", seed, V, 1, d, std=w_std)[:, 0]
    dloss = (rng.uniform(0.5, 1.5, src.size) / src.size).astype(np.float32)
    return T, src, tgt, h, w, dloss


def run(sp, T, src, tgt, h, w, dloss, d, V, dev, keep_logits=False):
    with torch.cuda.device(dev):
        edges = sp.EdgePlan(src, tgt, T, V)
    ht, wt = bf16_tensor(h, dev), bf16_tensor(w, dev)
    saved = torch.empty(edges.saved_bytes(), dtype=torch.uint8, device=dev) if keep_logits else None
    loss, lse = sp.edge_loss_fwd(ht, wt, edges, saved=saved)
    dh, dw = sp.edge_loss_bwd(ht, wt, edges, lse, torch.from_numpy(dloss).to(dev), saved=saved)
    torch.cuda.synchronize()
    return loss, lse, dh, dw


CASES = [
    # label, seed, max tokens, hidden, vocab, sampled fraction, weight std
    ("one_chunk", 41, 400, 128, 1000, 0.6, 0.1),
    ("three_chunks_ragged", 42, 500, 256, 20000, 0.5, 0.06),
    ("hidden_200", 43, 300, 200, 9000, 0.8, 0.08),
    ("one_edge", 44, 40, 64, 8192, 0.0, 0.1),
    ("odd_vocab_8201", 46, 300, 8, 8201, 0.5, 0.3),  # vocabulary not a multiple of 4: scalar row paths
]


@pytest.mark.parametrize("keep", [False, True], ids=["recompute", "saved_logits"])
@pytest.mark.parametrize("label,seed,Tm,d,V,p,ws", CASES, ids=[c[0] for c in CASES])
def test_edge_loss_matches_oracle(label, seed, Tm, d, V, p, ws, keep):
    """Both backward paths: logits recomputed per chunk, or kept by the
    forward as fp16 relative to each chunk's row maximum."""
    import shared_prefix_tree_amd as sp

    T, src, tgt, h, w, dloss = make_case(seed, Tm, d, V, p, ws)
    log(f"edge loss {label}: T={T} E={src.size} d={d} V={V} saved logits={keep}")
    dev = "cuda:0"
    loss, lse, dh, dw = run(sp, T, src, tgt, h, w, dloss, d, V, dev, keep)
    hf, wf = bf16_to_f32(h), bf16_to_f32(w)
    loss_ref, lse_ref = oracle.edge_loss_forward(hf, wf, src, tgt)
    dh_ref, dw_ref = oracle.edge_loss_backward(hf, wf, src, tgt, dloss)
    e_loss = float(np.abs(to_host(loss) - loss_ref).max())
    e_lse = float(np.abs(to_host(lse) - lse_ref).max())
    e_dh, e_dw = rel_l2(to_host(dh), dh_ref), rel_l2(to_host(dw), dw_ref)
    log(f"  loss max-abs {e_loss:.3g} lse max-abs {e_lse:.3g} dh rel-L2 {e_dh:.3g} dW rel-L2 {e_dw:.3g}")
    assert e_loss <= LOSS_TOL and e_lse <= LOSS_TOL
    assert e_dh <= GRAD_TOL and e_dw <= GRAD_TOL
    others = np.setdiff1d(np.arange(T), src)
    assert np.all(to_host(dh)[others] == 0.0)
    # bitwise reproducible
    loss2, lse2, dh2, dw2 = run(sp, T, src, tgt, h, w, dloss, d, V, dev, keep)
    for a, b in ((loss, loss2), (lse, lse2), (dh, dh2), (dw, dw2)):
        assert torch.equal(a, b)


def test_edge_loss_full_vocabulary_and_width():
    """A 4096-wide hidden state and a 131,072-word vocabulary (16 chunks):
    every output against the oracle, on 48 edges of a small tree (saved
    logits, as the benchmark runs)."""
    import shared_prefix_tree_amd as sp

    d, V = 4096, 131072
    rng = np.random.default_rng(45)
    topo = random_forest(rng, max_tokens=120, max_len=20, max_depth=4, p_new_root=0.0)
    T = topo.total_tokens
    src, tgt = sampled_edges(topo, rng, V, 1.0)
    src, tgt = src[:48], tgt[:48]
    h = make_tensor("hidden", 45, T, 1, d)[:, 0]
    w = make_tensor("weight", 45, V, 1, d, std=0.02)[:, 0]
    dloss = np.full(src.size, 1.0 / src.size, np.float32)
    log(f"edge loss full vocabulary: T={T} E={src.size} d={d} V={V}")
    loss, lse, dh, dw = run(sp, T, src, tgt, h, w, dloss, d, V, "cuda:0", keep_logits=True)
    hf, wf = bf16_to_f32(h), bf16_to_f32(w)
    loss_ref, lse_ref = oracle.edge_loss_forward(hf, wf, src, tgt)
    dh_ref, dw_ref = oracle.edge_loss_backward(hf, wf, src, tgt, dloss)
    e = (float(np.abs(to_host(loss) - loss_ref).max()), float(np.abs(to_host(lse) - lse_ref).max()),
         rel_l2(to_host(dh), dh_ref), rel_l2(to_host(dw), dw_ref))
    log(f"  loss {e[0]:.3g} lse {e[1]:.3g} dh {e[2]:.3g} dW {e[3]:.3g}")
    assert e[0] <= LOSS_TOL and e[1] <= LOSS_TOL and e[2] <= GRAD_TOL and e[3] <= GRAD_TOL


def test_edge_loss_rejects_bad_hidden_size():
    import shared_prefix_tree_amd as sp

    dev = "cuda:0"
    with torch.cuda.device(dev):
        edges = sp.EdgePlan(np.array([0], np.int32), np.array([1], np.int32), 2, 16)
    h = torch.zeros(2, 12, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(16, 12, dtype=torch.bfloat16, device=dev)
    with pytest.raises(Exception, match="multiple of 8"):
        sp.edge_loss_fwd(h, w, edges)
