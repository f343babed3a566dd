"""Pins of the sampled-edge loss oracle against facts fixed independently of
it: closed forms, a library log-sum-exp, brute-force logits, invariances of
the softmax cross-entropy and finite differences of the loss."""

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from workloads import random_forest, sampled_edges


def tiny(rng, T=6, d=3, V=5, E=8):
    h = rng.standard_normal((T, d))
    w = rng.standard_normal((V, d))
    src = rng.integers(0, T, E)
    src[1] = src[0]  # a branch point: one source, two edges
    tgt = rng.integers(0, V, E)
    dloss = rng.uniform(0.5, 2.0, E)
    return h, w, src, tgt, dloss


def test_logits_brute_force():
    rng = np.random.default_rng(1)
    h, w, src, tgt, _ = tiny(rng)
    z = oracle.edge_logits(h, w, src)
    for e in range(len(src)):
        for v in range(w.shape[0]):
            ref = sum(w[v, c] * h[src[e], c] for c in range(h.shape[1]))
            assert abs(z[e, v] - ref) < 1e-12


def test_zero_weight_gives_log_vocab():
    rng = np.random.default_rng(2)
    h, w, src, tgt, dloss = tiny(rng, V=7)
    w[:] = 0.0
    loss, lse = oracle.edge_loss_forward(h, w, src, tgt)
    assert np.allclose(loss, np.log(7.0), rtol=0, atol=1e-15)
    assert np.allclose(lse, np.log(7.0), rtol=0, atol=1e-15)
    dh, dw = oracle.edge_loss_backward(h, w, src, tgt, dloss)
    assert np.all(dh == 0.0)
    # uniform softmax: row v of dW is sum_e (1/V - [v == tgt_e]) dloss_e h[src_e]
    for v in range(7):
        ref = np.zeros(h.shape[1])
        for e in range(len(src)):
            ref += (1.0 / 7.0 - (1.0 if tgt[e] == v else 0.0)) * dloss[e] * h[src[e]]
        assert np.allclose(dw[v], ref, rtol=0, atol=1e-13)


def test_two_word_vocabulary_is_softplus():
    rng = np.random.default_rng(3)
    h, w, src, tgt, _ = tiny(rng, V=2)
    w *= 300.0  # large margins: the max shift must keep it finite
    loss, _ = oracle.edge_loss_forward(h, w, src, tgt)
    for e in range(len(src)):
        zt = float(w[tgt[e]] @ h[src[e]])
        zo = float(w[1 - tgt[e]] @ h[src[e]])
        assert np.isfinite(loss[e])
        assert abs(loss[e] - np.logaddexp(0.0, zo - zt)) <= 1e-12 * max(1.0, abs(loss[e]))


def test_lse_matches_scipy_and_loss_is_nonnegative():
    rng = np.random.default_rng(4)
    h, w, src, tgt, _ = tiny(rng, T=20, d=16, V=300, E=40)
    loss, lse = oracle.edge_loss_forward(h, w, src, tgt)
    z = np.array([[w[v] @ h[s] for v in range(300)] for s in src])
    assert np.allclose(lse, logsumexp(z, axis=1), rtol=1e-14, atol=1e-13)
    assert np.all(loss >= 0.0)


def test_shift_of_every_vocabulary_row_changes_nothing():
    rng = np.random.default_rng(5)
    h, w, src, tgt, _ = tiny(rng)
    c = rng.standard_normal(h.shape[1])
    a, _ = oracle.edge_loss_forward(h, w, src, tgt)
    b, _ = oracle.edge_loss_forward(h, w + c[None, :], src, tgt)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_dw_sums_to_zero_over_the_vocabulary_and_unsourced_rows_are_zero():
    rng = np.random.default_rng(6)
    h, w, src, tgt, dloss = tiny(rng, T=10)
    dh, dw = oracle.edge_loss_backward(h, w, src, tgt, dloss)
    assert np.allclose(dw.sum(axis=0), 0.0, atol=1e-13)
    others = np.setdiff1d(np.arange(10), src)
    assert others.size and np.all(dh[others] == 0.0)


def test_finite_differences():
    rng = np.random.default_rng(7)
    h, w, src, tgt, dloss = tiny(rng)

    def total(hh, ww):
        return float(oracle.edge_loss_forward(hh, ww, src, tgt)[0] @ dloss)

    dh, dw = oracle.edge_loss_backward(h, w, src, tgt, dloss)
    eps = 1e-6
    for x, g in ((h, dh), (w, dw)):
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            up = total(h, w)
            x[idx] = old - eps
            dn = total(h, w)
            x[idx] = old
            assert abs((up - dn) / (2 * eps) - g[idx]) < 1e-7, idx


def test_one_loss_owner_per_action():
    """An edge listed twice with its weight halved is the same action: the
    gradients do not change."""
    rng = np.random.default_rng(8)
    h, w, src, tgt, dloss = tiny(rng)
    dh, dw = oracle.edge_loss_backward(h, w, src, tgt, dloss)
    src2 = np.concatenate([src, src[:3]])
    tgt2 = np.concatenate([tgt, tgt[:3]])
    dl2 = np.concatenate([dloss, dloss[:3] / 2])
    dl2[:3] /= 2
    dh2, dw2 = oracle.edge_loss_backward(h, w, src2, tgt2, dl2)
    assert np.allclose(dh, dh2, atol=1e-13) and np.allclose(dw, dw2, atol=1e-13)


def test_sampled_edges_follow_the_tree():
    rng = np.random.default_rng(9)
    topo = random_forest(rng, max_tokens=300, max_len=40, max_depth=4)
    src, tgt = sampled_edges(topo, rng, vocab=50, p_sampled=1.0)
    T = topo.total_tokens
    # every token except a root's first one is a sampled action; each edge's
    # source is the token right before it in its sequence
    roots = topo.seg_start[topo.parent < 0]
    assert src.size == T - roots.size
    assert np.all((src >= 0) & (src < T)) and np.all((tgt >= 0) & (tgt < 50))
    for s in range(topo.num_segments):
        p = topo.parent[s]
        if p >= 0:
            assert (src == topo.seg_start[p] + topo.seg_len[p] - 1).sum() >= 1
