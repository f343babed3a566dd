"""Pins for the CPU oracle, each against something other than the oracle.

* golden hand-derived rational examples (tests/golden/);
* closed forms: q = 0 gives uniform attention over the visible set, constant v
  gives constant output, one-hot v reads the visible set off the output;
* reconstructed root-to-leaf sequences run through torch's float64
  scaled-dot-product attention (a library routine) -- the correctness
  reference named in Megatron-LM issue "Shared-prefix training with context
  parallelism for exact agent trajectories", section "Describe alternatives
  you've considered", item 1 (independent exact-call sequences);
* central finite differences of L = sum <dout, out>;
* sibling-permutation and fragment-copy invariance;
* brute force on tiny forests.

The visible sets used as expectations are derived here from children lists
(root-to-leaf enumeration), not from the oracle's parent walk.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import Topology, fragment_forest, random_forest, tiny_tree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent helpers (children lists, reconstructed sequences)


def children_lists(topo):
    ch = [[] for _ in range(topo.num_segments)]
    roots = []
    for s, p in enumerate(topo.parent):
        (roots if p < 0 else ch[p]).append(s)
    return roots, ch


def root_to_leaf_sequences(topo):
    """Token lists of every root-to-leaf sequence, leaves in DFS order."""
    roots, ch = children_lists(topo)
    seqs = []

    def walk(s, prefix):
        toks = prefix + list(range(int(topo.seg_start[s]), int(topo.seg_start[s] + topo.seg_len[s])))
        if not ch[s]:
            seqs.append(toks)
        for c in ch[s]:
            walk(c, toks)

    for r in roots:
        walk(r, [])
    return seqs


def visible_from_sequences(topo):
    """V(i) as the prefix (inclusive) of any reconstructed sequence holding i."""
    vis = {}
    for seq in root_to_leaf_sequences(topo):
        for p, t in enumerate(seq):
            vis.setdefault(t, set(seq[: p + 1]))
            assert vis[t] == set(seq[: p + 1])  # every copy has the same context
    return vis


def sdpa_on_sequences(q, k, v, dout, topo, scale=None):
    """Dense causal attention (torch, float64) on every reconstructed sequence.

    Returns per-token out/lse from the sequences and the tree gradients:
    dq from the owner copy (first sequence holding the token), dk/dv summed
    over all copies, with dout given to the owner copy only.
    """
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((Hq, T), np.nan)
    dq = np.zeros((T, Hq, D))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    owner = {}
    for n, seq in enumerate(root_to_leaf_sequences(topo)):
        for t in seq:
            owner.setdefault(t, n)
    for n, seq in enumerate(root_to_leaf_sequences(topo)):
        idx = torch.tensor(seq)
        Q = torch.tensor(q)[idx].permute(1, 0, 2).contiguous().requires_grad_(True)
        K = torch.tensor(k)[idx].permute(1, 0, 2).contiguous().requires_grad_(True)
        V = torch.tensor(v)[idx].permute(1, 0, 2).contiguous().requires_grad_(True)
        Kr = K.repeat_interleave(G, dim=0)
        Vr = V.repeat_interleave(G, dim=0)
        O = torch.nn.functional.scaled_dot_product_attention(
            Q[None], Kr[None], Vr[None], is_causal=True, scale=scale
        )[0]
        own = torch.tensor([owner[t] == n for t in seq], dtype=torch.float64)
        dO = torch.tensor(dout)[idx].permute(1, 0, 2) * own[None, :, None]
        (O * dO).sum().backward()
        L = len(seq)
        S = scale * Q.detach() @ Kr.detach().transpose(1, 2)
        S = S.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
        lse_seq = torch.logsumexp(S, dim=-1)
        for p, t in enumerate(seq):
            out[t] = O[:, p].detach().numpy()
            lse[:, t] = lse_seq[:, p].numpy()
            if owner[t] == n:
                dq[t] = Q.grad[:, p].numpy()
            dk[t] += K.grad[:, p].numpy()
            dv[t] += V.grad[:, p].numpy()
    return out, lse, dq, dk, dv


def rand_inputs(rng, T, Hq, Hkv, D, std=1.0):
    return (
        rng.standard_normal((T, Hq, D)) * std,
        rng.standard_normal((T, Hkv, D)) * std,
        rng.standard_normal((T, Hkv, D)) * std,
        rng.standard_normal((T, Hq, D)),
    )


def small_forests(n, seed=0, **kw):
    rng = np.random.default_rng(seed)
    return [random_forest(rng, **kw) for _ in range(n)]


# ---------------------------------------------------------------------------
# golden hand-derived examples


def _parse_value(tok):
    if "ln(" in tok:
        coef, _, rest = tok.partition("ln(")
        coef = coef.rstrip("*")
        c = Fraction(coef) if coef not in ("", "+") else Fraction(1)
        if coef == "-":
            c = Fraction(-1)
        return float(c) * math.log(int(rest.rstrip(")")))
    return float(Fraction(tok))


def load_golden(name):
    fields = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, vals = line.partition(":")
            fields[key.strip()] = vals.split()
    topo = Topology(
        [int(x) for x in fields["parent"]],
        [int(x) for x in fields["seg_start"]],
        [int(x) for x in fields["seg_len"]],
    )
    arr = {k: np.array([_parse_value(x) for x in v]) for k, v in fields.items() if k not in ("parent", "seg_start", "seg_len")}
    return topo, arr


@pytest.mark.parametrize("name", ["tree5_uniform_scores.txt", "tree5_weighted_scores.txt"])
def test_golden_examples(name):
    topo, g = load_golden(name)
    col = lambda x: x.reshape(-1, 1, 1)  # noqa: E731  [T, 1 head, D=1]
    q, k, v, dout = col(g["q"]), col(g["k"]), col(g["v"]), col(g["dout"])
    scale = float(g["scale"][0])
    out, lse = oracle.forward(q, k, v, topo, scale)
    np.testing.assert_allclose(out[:, 0, 0], g["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], g["lse"], rtol=0, atol=1e-14)
    dq, dk, dv = oracle.backward(q, k, v, dout, topo, scale)
    np.testing.assert_allclose(dq[:, 0, 0], g["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk[:, 0, 0], g["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv[:, 0, 0], g["dv"], rtol=0, atol=1e-14)
    # the dense brute force and the sampled forms agree with the same values
    out2, lse2 = oracle.masked_dense_forward(q, k, v, topo, scale)
    np.testing.assert_allclose(out2[:, 0, 0], g["out"], atol=1e-14)
    dq2, dk2, dv2 = oracle.masked_dense_backward(q, k, v, dout, topo, scale)
    np.testing.assert_allclose(dk2[:, 0, 0], g["dk"], atol=1e-14)
    np.testing.assert_allclose(dv2[:, 0, 0], g["dv"], atol=1e-14)
    rows = np.arange(5)
    o3, l3 = oracle.forward_rows(q, k, v, topo, rows, scale)
    np.testing.assert_allclose(o3[:, 0, 0], g["out"], atol=1e-14)
    np.testing.assert_allclose(oracle.backward_rows(q, k, v, dout, topo, rows, scale)[:, 0, 0], g["dq"], atol=1e-14)
    dk4, dv4 = oracle.backward_keys(q, k, v, dout, topo, rows, 0, scale)
    np.testing.assert_allclose(dk4[:, 0], g["dk"], atol=1e-14)
    np.testing.assert_allclose(dv4[:, 0], g["dv"], atol=1e-14)


def test_pairs_tiny_tree_by_hand():
    # root 64 tokens: 64*65/2 pairs; each of 4 children of 32 tokens sees the
    # whole root (32*64) plus its own causal triangle (32*33/2).
    assert oracle.pairs(tiny_tree()) == 64 * 65 // 2 + 4 * (32 * 64 + 32 * 33 // 2) == 12384


def test_pairs_brute_force():
    for topo in small_forests(20, seed=3, max_tokens=60):
        vis = visible_from_sequences(topo)
        assert oracle.pairs(topo) == sum(len(s) for s in vis.values())


# ---------------------------------------------------------------------------
# visible set / closed forms


def test_visible_sets_match_reconstructed_sequences():
    for topo in small_forests(30, seed=1, max_tokens=50) + [tiny_tree(8, 4, 3)]:
        vis = visible_from_sequences(topo)
        assert sorted(vis) == list(range(topo.total_tokens))
        for i in range(topo.total_tokens):
            assert set(oracle.visible_tokens(topo, i).tolist()) == vis[i]
            assert oracle.position_in_sequence(topo, i) == len(vis[i]) - 1


def test_ancestors_subtree_end_and_segment_pairs_from_children_lists():
    # expectations from the children lists alone: the root-to-segment path of a
    # DFS walk, the last token the walk emits under a segment, and the pairs of
    # a segment's tokens counted from their reconstructed prefixes
    for topo in small_forests(25, seed=12, max_tokens=70) + [tiny_tree(8, 4, 3)]:
        roots, ch = children_lists(topo)
        path_of, last_of = {}, {}

        def walk(s, path):
            path_of[s] = list(path)
            last = int(topo.seg_start[s] + topo.seg_len[s])
            for c in ch[s]:
                last = max(last, walk(c, path + [s]))
            last_of[s] = last
            return last

        for r in roots:
            walk(r, [])
        vis = visible_from_sequences(topo)
        per_seg = oracle.segment_pairs(topo)
        end = oracle.subtree_end(topo)
        for s in range(topo.num_segments):
            assert list(oracle.ancestors(np.asarray(topo.parent), s)) == path_of[s]
            assert int(end[s]) == last_of[s]
            toks = range(int(topo.seg_start[s]), int(topo.seg_start[s] + topo.seg_len[s]))
            assert per_seg[s] == sum(len(vis[t]) for t in toks)


def test_mask_form_subtree_interval():
    # j visible from i  <=>  j <= i and i < subtree_end(seg(j)), because a DFS
    # pre-order keeps every subtree contiguous.
    for topo in small_forests(20, seed=2, max_tokens=50):
        m = oracle.visible_mask(topo)
        end = oracle.subtree_end(topo)
        seg = np.repeat(np.arange(topo.num_segments), topo.seg_len)
        T = topo.total_tokens
        i, j = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
        assert np.array_equal(m, (j <= i) & (i < end[seg[j]]))


def test_zero_query_one_hot_values_read_off_mask():
    for topo in small_forests(10, seed=4, max_tokens=40):
        T = topo.total_tokens
        vis = visible_from_sequences(topo)
        q = np.zeros((T, 1, T))
        k = np.random.default_rng(0).standard_normal((T, 1, T))
        v = np.eye(T).reshape(T, 1, T)
        out, lse = oracle.forward(q, k, v, topo)
        for i in range(T):
            expect = np.zeros(T)
            expect[list(vis[i])] = 1.0 / len(vis[i])
            np.testing.assert_allclose(out[i, 0], expect, atol=1e-15)
            assert abs(lse[0, i] - math.log(len(vis[i]))) < 1e-13


def test_zero_query_closed_form_gradient_dv():
    # q = 0: P_ij = 1/|V(i)|, so dv_j = sum_{i sees j} dout_i / |V(i)|.
    for topo in small_forests(5, seed=5, max_tokens=40):
        T = topo.total_tokens
        vis = visible_from_sequences(topo)
        rng = np.random.default_rng(1)
        q = np.zeros((T, 2, 3))
        k, v = rng.standard_normal((T, 1, 3)), rng.standard_normal((T, 1, 3))
        dout = rng.standard_normal((T, 2, 3))
        _, _, dv = oracle.backward(q, k, v, dout, topo)
        expect = np.zeros((T, 1, 3))
        for i in range(T):
            for j in vis[i]:
                expect[j, 0] += dout[i].sum(axis=0) / len(vis[i])
        np.testing.assert_allclose(dv, expect, atol=1e-13)


def test_constant_values_give_constant_output():
    topo = small_forests(1, seed=6, max_tokens=50)[0]
    T = topo.total_tokens
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((T, 4, 5)), rng.standard_normal((T, 2, 5))
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0, 7.0]), (T, 2, 5)).copy()
    out, _ = oracle.forward(q, k, v, topo)
    np.testing.assert_allclose(out, np.broadcast_to(v[:, :1], out.shape), atol=1e-13)


def test_stored_bf16_output_gradient_by_hand():
    # One segment of three tokens, D = 1, q = 0 (so every visible key has the
    # same score), k = (1, 2, 4), v = (0, 0, 1), dout = (0, 0, 1).  Token 2
    # sees all three keys with P = 1/3: out_2 = 1/3, dP_2j = v_j, and
    #   dq_2 = sum_j P (v_j - delta) k_j = (4 - 7 delta) / 3.
    # Exact delta = 1/3 gives 5/9; the bfloat16-stored output rounds 1/3 to
    # 171/512 (0.0101010101... to 8 significant bits, to nearest), so
    # delta = 171/512 and dq_2 = (4 - 1197/512) / 3 = 851/1536.
    topo = Topology([-1], [0], [3])
    q = np.zeros((3, 1, 1))
    k = np.array([1.0, 2.0, 4.0]).reshape(3, 1, 1)
    v = np.array([0.0, 0.0, 1.0]).reshape(3, 1, 1)
    dout = np.array([0.0, 0.0, 1.0]).reshape(3, 1, 1)
    dq, dk, dv = oracle.backward(q, k, v, dout, topo)
    assert dq[2, 0, 0] == pytest.approx(5 / 9, abs=1e-15)
    dq_b, dk_b, dv_b = oracle.backward(q, k, v, dout, topo, out_dtype="bf16")
    assert dq_b[2, 0, 0] == pytest.approx(851 / 1536, abs=1e-15)
    # dv does not use the row statistic; dk_j = sum_i dS_ij q_i = 0 (q = 0)
    np.testing.assert_array_equal(dv_b, dv)
    np.testing.assert_array_equal(dk_b, dk)


def test_stored_bf16_output_is_exact_where_representable():
    # Constant values that bfloat16 holds exactly make every output exact,
    # so the stored-output mode must return the exact gradients bit for bit.
    topo = small_forests(1, seed=8, max_tokens=40)[0]
    T = topo.total_tokens
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((T, 2, 4)), rng.standard_normal((T, 1, 4))
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0]), (T, 1, 4)).copy()
    dout = rng.standard_normal((T, 2, 4))
    exact = oracle.backward(q, k, v, dout, topo)
    stored = oracle.backward(q, k, v, dout, topo, out_dtype="bf16")
    for a, b in zip(exact, stored):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# reconstructed sequences vs torch SDPA (forward and one-owner backward)


CASES = [
    ("tiny_tree", tiny_tree(), 1, 1, 64),
    ("single_segment", Topology([-1], [0], [37]), 2, 1, 8),
    ("chain", Topology([-1, 0, 1, 2], [0, 5, 12, 13], [5, 7, 1, 9]), 4, 2, 8),
    ("star", Topology([-1, 0, 0, 0], [0, 9, 12, 20], [9, 3, 8, 1]), 4, 1, 8),
]


@pytest.mark.parametrize("name,topo,Hq,Hkv,D", CASES, ids=[c[0] for c in CASES])
def test_special_cases_equal_sdpa(name, topo, Hq, Hkv, D):
    rng = np.random.default_rng(7)
    q, k, v, dout = rand_inputs(rng, topo.total_tokens, Hq, Hkv, D)
    ref = sdpa_on_sequences(q, k, v, dout, topo)
    out, lse = oracle.forward(q, k, v, topo)
    np.testing.assert_allclose(out, ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref[1], rtol=0, atol=1e-12)
    dq, dk, dv = oracle.backward(q, k, v, dout, topo)
    np.testing.assert_allclose(dq, ref[2], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, ref[3], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, ref[4], rtol=0, atol=1e-11)


def test_random_forests_equal_sdpa_and_brute_force():
    for n, topo in enumerate(small_forests(12, seed=8, max_tokens=64)):
        rng = np.random.default_rng(100 + n)
        Hq, Hkv = [(1, 1), (2, 1), (4, 2), (4, 4)][n % 4]
        q, k, v, dout = rand_inputs(rng, topo.total_tokens, Hq, Hkv, 6, std=1.5)
        ref = sdpa_on_sequences(q, k, v, dout, topo)
        out, lse = oracle.forward(q, k, v, topo)
        dq, dk, dv = oracle.backward(q, k, v, dout, topo)
        for got, want in zip((out, lse, dq, dk, dv), ref):
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)
        bf = oracle.masked_dense_backward(q, k, v, dout, topo)
        for got, want in zip((dq, dk, dv), bf):
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# finite differences


def test_gradients_match_central_differences():
    rng = np.random.default_rng(9)
    topo = random_forest(rng, max_tokens=20, max_len=6, max_depth=3)
    T = topo.total_tokens
    q, k, v, dout = rand_inputs(rng, T, 2, 1, 3)
    dq, dk, dv = oracle.backward(q, k, v, dout, topo)

    def loss(q_, k_, v_):
        return float((oracle.forward(q_, k_, v_, topo)[0] * dout).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=name)


# ---------------------------------------------------------------------------
# invariances


def relinearize(topo, rng):
    """Re-emit the forest in DFS order with every child list shuffled.

    Returns (new topology, perm) with new token t' holding old token perm[t']."""
    roots, ch = children_lists(topo)
    nodes, perm = [], []

    def emit(s, par):
        me = len(nodes)
        nodes.append((par, int(topo.seg_len[s])))
        perm.extend(range(int(topo.seg_start[s]), int(topo.seg_start[s] + topo.seg_len[s])))
        kids = list(ch[s])
        rng.shuffle(kids)
        for c in kids:
            emit(c, me)

    rs = list(roots)
    rng.shuffle(rs)
    for r in rs:
        emit(r, -1)
    parent = [p for p, _ in nodes]
    seg_len = [n for _, n in nodes]
    seg_start = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
    return Topology(parent, seg_start, seg_len), np.array(perm)


def test_sibling_permutation_invariance():
    for n, topo in enumerate(small_forests(6, seed=10, max_tokens=64)):
        rng = np.random.default_rng(n)
        new, perm = relinearize(topo, rng)
        q, k, v, dout = rand_inputs(rng, topo.total_tokens, 2, 1, 4)
        out, lse = oracle.forward(q, k, v, topo)
        dq, dk, dv = oracle.backward(q, k, v, dout, topo)
        out2, lse2 = oracle.forward(q[perm], k[perm], v[perm], new)
        dq2, dk2, dv2 = oracle.backward(q[perm], k[perm], v[perm], dout[perm], new)
        np.testing.assert_allclose(out2, out[perm], atol=1e-12)
        np.testing.assert_allclose(lse2, lse[:, perm], atol=1e-12)
        for a, b in ((dq2, dq), (dk2, dk), (dv2, dv)):
            np.testing.assert_allclose(a, b[perm], atol=1e-11)


def test_fragment_copy_invariance():
    rng = np.random.default_rng(11)
    topo = fragment_forest(rng, fragments=3, capacity=120, lo=4, hi=30, max_depth=3)
    logical = topo.logical
    src = topo.source
    L = logical.total_tokens
    q, k, v, dout = rand_inputs(np.random.default_rng(12), L, 4, 2, 5)
    first = np.zeros(len(src), dtype=bool)
    _, first_idx = np.unique(src, return_index=True)
    first[first_idx] = True  # the loss owner of each logical token
    out_l, lse_l = oracle.forward(q, k, v, logical)
    dq_l, dk_l, dv_l = oracle.backward(q, k, v, dout, logical)
    out_p, lse_p = oracle.forward(q[src], k[src], v[src], topo)
    dq_p, dk_p, dv_p = oracle.backward(q[src], k[src], v[src], dout[src] * first[:, None, None], topo)
    np.testing.assert_allclose(out_p, out_l[src], atol=1e-12)
    np.testing.assert_allclose(lse_p, lse_l[:, src], atol=1e-12)
    np.testing.assert_allclose(dq_p[first], dq_l[src[first]], atol=1e-11)
    np.testing.assert_allclose(dq_p[~first], 0.0, atol=0)
    for grad_p, grad_l in ((dk_p, dk_l), (dv_p, dv_l)):
        summed = np.zeros_like(grad_l)
        np.add.at(summed, src, grad_p)
        np.testing.assert_allclose(summed, grad_l, atol=1e-11)


# ---------------------------------------------------------------------------
# sampled forms agree with the full forms


def test_sampled_forms_agree_with_full():
    rng = np.random.default_rng(13)
    topo = random_forest(rng, max_tokens=120, max_len=20, max_depth=4)
    T = topo.total_tokens
    q, k, v, dout = rand_inputs(rng, T, 4, 2, 8)
    out, lse = oracle.forward(q, k, v, topo)
    dq, dk, dv = oracle.backward(q, k, v, dout, topo)
    rows = rng.choice(T, size=min(T, 17), replace=False)
    o, l = oracle.forward_rows(q, k, v, topo, rows)
    np.testing.assert_allclose(o, out[rows], atol=1e-12)
    np.testing.assert_allclose(l, lse[:, rows], atol=1e-12)
    np.testing.assert_allclose(oracle.backward_rows(q, k, v, dout, topo, rows), dq[rows], atol=1e-11)
    for g in range(2):
        dk_s, dv_s = oracle.backward_keys(q, k, v, dout, topo, rows, g)
        np.testing.assert_allclose(dk_s, dk[rows, g], atol=1e-11)
        np.testing.assert_allclose(dv_s, dv[rows, g], atol=1e-11)
    # head / segment restriction leaves the selected entries unchanged
    o2, l2 = oracle.forward(q, k, v, topo, heads=[1, 2], segments=[0])
    sl = slice(int(topo.seg_start[0]), int(topo.seg_start[0] + topo.seg_len[0]))
    np.testing.assert_allclose(o2[sl, 1:3], out[sl, 1:3], atol=1e-13)
    dq3, dk3, dv3 = oracle.backward(q, k, v, dout, topo, kv_heads=[1])
    np.testing.assert_allclose(dk3[:, 1], dk[:, 1], atol=1e-12)
    np.testing.assert_allclose(dq3[:, 2:4], dq[:, 2:4], atol=1e-12)
