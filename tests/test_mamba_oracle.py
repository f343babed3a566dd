"""Pins of the Mamba state-forking oracle against facts fixed independently
of its recurrence: the quadratic (state-space dual) form, plain chain runs
of every root-to-leaf sequence, numpy.convolve, finite differences, and the
one-owner sum over sequence copies."""

import numpy as np
import pytest

import oracle
from workloads import Topology, random_forest, tiny_tree


def inputs(rng, T, H=2, G=1, P=3, N=4, C=5, W=4):
    return dict(
        x=rng.standard_normal((T, H, P)),
        dt=rng.uniform(0.05, 0.6, (T, H)),
        A=-rng.uniform(0.5, 2.0, H),
        B=rng.standard_normal((T, G, N)),
        C=rng.standard_normal((T, G, N)),
        D=rng.standard_normal(H),
        cx=rng.standard_normal((T, C)),
        cw=rng.standard_normal((C, W)),
        cb=rng.standard_normal(C),
    )


def small_tree(rng):
    return random_forest(rng, max_tokens=40, max_len=6, max_depth=3, p_new_root=0.1)


def leaf_paths(topo):
    """(token list, leaf segment) for every root-to-leaf sequence."""
    S = topo.num_segments
    has_child = np.zeros(S, bool)
    has_child[topo.parent[topo.parent >= 0]] = True
    out = []
    for s in range(S):
        if has_child[s]:
            continue
        chain, a = [], s
        while a >= 0:
            chain.append(a)
            a = topo.parent[a]
        toks = np.concatenate([np.arange(topo.seg_start[c], topo.seg_start[c] + topo.seg_len[c]) for c in chain[::-1]])
        out.append((toks, s))
    return out


def chain_topo(n):
    return Topology(np.array([-1]), np.array([0]), np.array([n]))


def test_previous_token_on_the_tiny_tree():
    prev = oracle.previous_token(tiny_tree())
    assert prev[0] == -1 and prev[1] == 0 and prev[63] == 62
    for c in range(4):  # every branch continues from the root's last token
        first = 64 + 32 * c
        assert prev[first] == 63 and prev[first + 1] == first


def test_recurrence_equals_quadratic_form():
    rng = np.random.default_rng(1)
    topo = small_tree(rng)
    d = inputs(rng, topo.total_tokens, H=4, G=2)
    y = oracle.ssm_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], topo)
    T, H, P = d["x"].shape
    for i in range(T):
        path = [int(j) for j in oracle.visible_tokens(topo, i)]  # ancestor path and i, in order
        for h in range(H):
            g = h // 2
            ref = d["D"][h] * d["x"][i, h]
            for pos, j in enumerate(path):
                decay = np.exp(d["A"][h] * sum(d["dt"][k, h] for k in path[pos + 1:]))
                ref = ref + decay * float(d["C"][i, g] @ d["B"][j, g]) * d["dt"][j, h] * d["x"][j, h]
            assert np.allclose(y[i, h], ref, rtol=1e-11, atol=1e-12), (i, h)


def test_every_sequence_equals_a_plain_chain_run():
    rng = np.random.default_rng(2)
    topo = small_tree(rng)
    d = inputs(rng, topo.total_tokens)
    y = oracle.ssm_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], topo)
    cy = oracle.conv_forward(d["cx"], d["cw"], d["cb"], topo)
    for toks, _ in leaf_paths(topo):
        n = toks.size
        yc = oracle.ssm_forward(d["x"][toks], d["dt"][toks], d["A"], d["B"][toks], d["C"][toks], d["D"], chain_topo(n))
        assert np.allclose(y[toks], yc, rtol=1e-12, atol=1e-12)
        for c in range(d["cx"].shape[1]):  # causal convolution of the sequence
            ref = np.convolve(d["cx"][toks, c], d["cw"][c, ::-1])[:n] + d["cb"][c]
            assert np.allclose(cy[toks, c], ref, rtol=1e-12, atol=1e-12)


def test_finite_differences():
    rng = np.random.default_rng(3)
    topo = Topology(np.array([-1, 0, 1, 0]), np.array([0, 3, 5, 7]), np.array([3, 2, 2, 3]))
    d = inputs(rng, topo.total_tokens, H=2, G=1, P=2, N=3, C=2, W=3)
    dy = rng.standard_normal(d["x"].shape)
    dcy = rng.standard_normal(d["cx"].shape)
    keys = ("x", "dt", "A", "B", "C", "D")

    def loss():
        y = oracle.ssm_forward(*(d[k] for k in keys), topo)
        cy = oracle.conv_forward(d["cx"], d["cw"], d["cb"], topo)
        return float((y * dy).sum() + (cy * dcy).sum())

    grads = dict(zip(keys, oracle.ssm_backward(dy, *(d[k] for k in keys), topo)))
    grads.update(zip(("cx", "cw", "cb"), oracle.conv_backward(dcy, d["cx"], d["cw"], topo)))
    eps = 1e-6
    for k, g in grads.items():
        x = d[k]
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            up = loss()
            x[idx] = old - eps
            dn = loss()
            x[idx] = old
            assert abs((up - dn) / (2 * eps) - g[idx]) < 1e-6 * max(1.0, abs(g[idx])), (k, idx)


def test_tree_gradients_are_sums_over_owned_copies():
    rng = np.random.default_rng(4)
    topo = small_tree(rng)
    d = inputs(rng, topo.total_tokens, H=4, G=2)
    T = topo.total_tokens
    dy = rng.standard_normal(d["x"].shape)
    dcy = rng.standard_normal(d["cx"].shape)
    keys = ("x", "dt", "A", "B", "C", "D")
    ref = oracle.ssm_backward(dy, *(d[k] for k in keys), topo)
    cref = oracle.conv_backward(dcy, d["cx"], d["cw"], topo)
    # a token's dy goes to the copy in the first leaf (DFS order) below its segment
    seg_of = np.repeat(np.arange(topo.num_segments), topo.seg_len)
    paths = leaf_paths(topo)
    leaves = [s for _, s in paths]
    owner = {}
    for t in range(T):
        owner[t] = min(s for s in leaves if s >= seg_of[t])
    acc = [np.zeros_like(r) for r in ref]
    cacc = [np.zeros_like(r) for r in cref]
    for toks, leaf in paths:
        mask = np.array([owner[t] == leaf for t in toks])
        dyc = dy[toks] * mask[:, None, None]
        dcyc = dcy[toks] * mask[:, None]
        n = toks.size
        got = oracle.ssm_backward(dyc, d["x"][toks], d["dt"][toks], d["A"], d["B"][toks], d["C"][toks], d["D"],
                                  chain_topo(n))
        for a, gv, per_token in zip(acc, got, (True, True, False, True, True, False)):
            if per_token:
                np.add.at(a, toks, gv)
            else:
                a += gv
        cg = oracle.conv_backward(dcyc, d["cx"][toks], d["cw"], chain_topo(n))
        np.add.at(cacc[0], toks, cg[0])
        cacc[1] += cg[1]
        cacc[2] += cg[2]
    for r, a in zip(ref + cref, acc + cacc):
        assert np.allclose(r, a, rtol=1e-10, atol=1e-10)
