"""Float64 CPU oracle of shared-prefix tree attention.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py``; never by the product path.  It
shares no code, constants or helpers with the HIP library.

What is computed, and where the pages define it
------------------------------------------------
Megatron-LM issue "Shared-prefix training with context parallelism for exact
agent trajectories":

* section "Describe the solution you'd like": tokens are packed as
  DFS-linearized segments with parent information, and attention for each
  query run is computed against only its ancestor path;
* section "Describe alternatives you've considered", item 1: independent
  exact-call sequences are the correctness reference.

Draft "feat(hybrid): add opt-in shared-prefix attention and Mamba execution"
(intro): prompt keys/values are reused while each suffix stays causally
isolated, and the backward pass accumulates every branch's contribution into
the shared prefix.

So for token i of segment u the visible key set is

    V(i) = (all tokens of every strict ancestor of u)
           + (tokens of u from its first token up to and including i),

and for query head h with key/value head g = h // (Hq / Hkv):

    S_ij = scale * <q[i,h], k[j,g]>              (scale = 1/sqrt(D) by default)
    out[i,h] = sum_{j in V(i)} softmax_j(S_i.) v[j,g]
    lse[h,i] = ln sum_{j in V(i)} exp(S_ij)       (natural log)

The backward pass is the exact gradient of L = sum_{i,h} <dout[i,h], out[i,h]>
(every tree token's upstream gradient counted once: one loss owner per token).

Readings where the pages are silent are listed in the design notes: the child
sees its whole parent segment, the diagonal is inclusive, the scale is
1/sqrt(D), query heads map to key/value heads in contiguous groups.

Array arithmetic runs in float64 on the CPU: NumPy for the tiny dense brute
force, PyTorch CPU ops (matmul, exp, max, sum) for the per-segment forms.

Parity status (pins live in ``tests/test_oracle.py``):

* ``visible_tokens`` / ``visible_mask`` -- pinned: hand-derived golden
  examples, Q=0 / one-hot-V read-off, equivalence with reconstructed
  root-to-leaf causal sequences.
* ``forward`` / ``forward_rows`` / ``masked_dense_forward`` -- pinned: golden
  rational examples, closed forms (Q=0, constant V), single segment and chain
  reduce to torch scaled-dot-product attention in float64, reconstructed
  sequence invariant, brute force on tiny forests.
* ``backward`` / ``backward_rows`` / ``backward_keys`` /
  ``masked_dense_backward`` -- pinned: golden rational gradients, central
  finite differences, torch autograd on reconstructed sequences with one loss
  owner per token, sibling-permutation and fragment-copy invariance.
  ``backward(..., out_dtype="bf16")`` (the row statistic taken from the
  output as a bfloat16 caller stores it) -- pinned: a hand-worked three-token
  gradient whose output 1/3 rounds to 171/512, and equality with the exact
  mode wherever the output is representable.
* ``pairs`` -- pinned: the tiny tree's count worked out by hand, and brute
  force (sum of |V(i)|).
* ``ancestors`` / ``subtree_end`` / ``segment_pairs`` /
  ``position_in_sequence`` -- pinned: root-to-segment paths, last emitted
  tokens and per-segment pair counts derived from children lists and
  reconstructed root-to-leaf sequences.

Every public function has a pin; none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np
import torch

# ---------------------------------------------------------------------------
# topology (definitions only; nothing here is tiled, merged or precomputed)


def _arrays(topo):
    return (
        np.asarray(topo.parent, dtype=np.int64),
        np.asarray(topo.seg_start, dtype=np.int64),
        np.asarray(topo.seg_len, dtype=np.int64),
    )


def ancestors(parent, s):
    """Strict ancestors of segment ``s``, root first, by walking parents."""
    out = []
    p = int(parent[s])
    while p >= 0:
        out.append(p)
        p = int(parent[p])
    return out[::-1]


def _segment_of_tokens(seg_start, seg_len):
    T = int(seg_start[-1] + seg_len[-1])
    seg = np.empty(T, dtype=np.int64)
    for s in range(len(seg_start)):
        seg[seg_start[s] : seg_start[s] + seg_len[s]] = s
    return seg


def visible_tokens(topo, i):
    """Token indices that token ``i`` may attend to: every token of each
    strict ancestor segment, then its own segment up to and including i."""
    parent, st, ln = _arrays(topo)
    u = int(_segment_of_tokens(st, ln)[i])
    parts = [np.arange(st[a], st[a] + ln[a]) for a in ancestors(parent, u)]
    parts.append(np.arange(st[u], i + 1))
    return np.concatenate(parts)


def visible_mask(topo):
    """Dense [T, T] boolean mask, row i = V(i).  Brute force, tiny inputs only."""
    _, st, ln = _arrays(topo)
    T = int(st[-1] + ln[-1])
    m = np.zeros((T, T), dtype=bool)
    for i in range(T):
        m[i, visible_tokens(topo, i)] = True
    return m


def position_in_sequence(topo, i):
    """Offset of token i in its reconstructed root-to-leaf sequence."""
    return len(visible_tokens(topo, i)) - 1


def subtree_end(topo):
    """One past the last token of each segment's subtree (by walking parents)."""
    parent, st, ln = _arrays(topo)
    S = len(parent)
    end = st + ln
    for s in range(S):
        for a in ancestors(parent, s):
            end[a] = max(end[a], st[s] + ln[s])
    return end


def _prefix_len(parent, ln, u):
    return int(sum(ln[a] for a in ancestors(parent, u)))


def segment_pairs(topo):
    """Per segment u: the (query, key) pairs of its queries, per head --
    each of its n tokens sees every ancestor token plus a causal prefix of u."""
    parent, st, ln = _arrays(topo)
    out = []
    for u in range(len(parent)):
        n = int(ln[u])
        out.append(n * _prefix_len(parent, ln, u) + n * (n + 1) // 2)
    return out


def pairs(topo):
    """Number of (query, key) pairs on ancestor paths, per head: sum_i |V(i)|."""
    return int(sum(segment_pairs(topo)))


# ---------------------------------------------------------------------------
# per-segment forward / backward (the plain definition, one segment at a time)


def _t(x):
    """Widen an input slice to a float64 CPU tensor.  Inputs may be float32
    (bf16 values are exact in float32) or float64 NumPy arrays; they are
    widened slice by slice so full-size tensors never need a float64 copy.
    All arithmetic is float64 (PyTorch CPU ops: matmul, exp, max, sum)."""
    return torch.as_tensor(np.asarray(x), dtype=torch.float64)


def _default_scale(D, scale):
    return 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)


def _path(parent, st, ln, u):
    """Key token indices for segment u: ancestors root->parent, then u."""
    idx = [np.arange(st[a], st[a] + ln[a]) for a in ancestors(parent, u)]
    idx.append(np.arange(st[u], st[u] + ln[u]))
    return np.concatenate(idx), _prefix_len(parent, ln, u)


def _row_chunks(n_rows, path_len, heads, budget=1 << 24):
    """Split a segment's query rows so one score block stays near ``budget``
    elements (memory bound only; the arithmetic is unchanged)."""
    step = max(1, budget // max(1, path_len * heads))
    return [(r, min(n_rows, r + step)) for r in range(0, n_rows, step)]


def _segment_scores(Q, Kp, scale, prefix, r0, r1):
    """scale * Q Kp^T with the own-segment causal rule applied.

    Q: [G, n, D] query rows r0..r1 of the segment for G heads; Kp: [P, D].
    Columns < prefix are ancestor keys (always visible); column c >= prefix
    is own-segment key c - prefix, visible iff c - prefix <= row offset.
    """
    S = scale * (Q @ Kp.T)
    cols = torch.arange(Kp.shape[0])
    rows = torch.arange(r0, r1)
    hidden = (cols[None, :] >= prefix) & (cols[None, :] - prefix > rows[:, None])
    return S.masked_fill(hidden[None], float("-inf"))


def forward(q, k, v, topo, scale=None, heads=None, segments=None):
    """Tree-attention forward.  Returns (out [T,Hq,D], lse [Hq,T]) in float64.

    ``heads`` / ``segments`` restrict the work to those query heads / query
    segments (other entries stay 0); used for bounded samples.
    """
    parent, st, ln = _arrays(topo)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(D, scale)
    heads = range(Hq) if heads is None else heads
    segments = range(len(parent)) if segments is None else segments
    out = np.zeros((T, Hq, D))
    lse = np.zeros((Hq, T))
    by_group = {}
    for h in heads:
        by_group.setdefault(h // G, []).append(h)
    for u in segments:
        idx, prefix = _path(parent, st, ln, u)
        s0, n = int(st[u]), int(ln[u])
        for g, hs in by_group.items():
            Kp, Vp = _t(k[idx, g]), _t(v[idx, g])
            for r0, r1 in _row_chunks(n, len(idx), len(hs)):
                Q = _t(q[s0 + r0 : s0 + r1][:, hs]).transpose(0, 1)
                S = _segment_scores(Q, Kp, scale, prefix, r0, r1)
                m = S.amax(dim=2, keepdim=True)
                E = torch.exp(S - m)
                l = E.sum(dim=2, keepdim=True)
                O = (E @ Vp) / l
                out[s0 + r0 : s0 + r1, hs] = O.transpose(0, 1).numpy()
                lse[hs, s0 + r0 : s0 + r1] = (m + torch.log(l))[..., 0].numpy()
    return out, lse


def _round_bf16(x):
    """x rounded to bfloat16 (through float32, to nearest even), as float64."""
    b = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32)).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


def backward(q, k, v, dout, topo, scale=None, kv_heads=None, segments=None, out_dtype=None):
    """Exact gradients (dq, dk, dv) of L = sum <dout, out>, float64.

    Each segment's contribution to its ancestors' dk/dv is added onto the
    shared prefix tokens: branch contributions accumulate there.
    ``kv_heads`` restricts the work to those key/value heads (and their
    query heads); ``segments`` to the contributions of those query segments
    (a bounded sample); other entries stay 0.

    The row statistic delta_i = sum_d dout[i,d] out[i,d] of the flash-style
    backward equals sum_j P_ij dP_ij for the exact output.  A backward that
    is handed the output as the caller stores it computes delta from that
    stored value; ``out_dtype="bf16"`` reproduces this by rounding the
    output to bfloat16 before delta (everything else stays exact).  Where
    the softmax is nearly one-hot, dS = P (dP - delta) cancels and dq is
    sensitive to that rounding.
    """
    parent, st, ln = _arrays(topo)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(D, scale)
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    segments = range(len(parent)) if segments is None else segments
    heads = [h for g in kv_heads for h in range(g * G, (g + 1) * G)]
    out, lse = forward(q, k, v, topo, scale, heads=heads, segments=segments)
    if out_dtype == "bf16":
        out = _round_bf16(out)
    elif out_dtype is not None:
        raise ValueError(f"out_dtype {out_dtype!r}: None or 'bf16'")
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for u in segments:
        idx, prefix = _path(parent, st, ln, u)
        s0, n = int(st[u]), int(ln[u])
        for g in kv_heads:
            hs = list(range(g * G, (g + 1) * G))
            Kp, Vp = _t(k[idx, g]), _t(v[idx, g])
            dKp = torch.zeros_like(Kp)
            dVp = torch.zeros_like(Vp)
            for r0, r1 in _row_chunks(n, len(idx), G):
                sl = slice(s0 + r0, s0 + r1)
                Q = _t(q[sl][:, hs]).transpose(0, 1)
                dO = _t(dout[sl][:, hs]).transpose(0, 1)
                O = _t(out[sl][:, hs]).transpose(0, 1)
                L = _t(lse[hs, sl])[..., None]
                S = _segment_scores(Q, Kp, scale, prefix, r0, r1)
                P = torch.exp(S - L)
                dVp += (P.transpose(1, 2) @ dO).sum(dim=0)
                dP = dO @ Vp.T
                delta = (dO * O).sum(dim=2, keepdim=True)
                dS = P * (dP - delta)
                dq[sl, hs] = (scale * (dS @ Kp)).transpose(0, 1).numpy()
                dKp += scale * (dS.transpose(1, 2) @ Q).sum(dim=0)
            dk[idx, g] += dKp.numpy()
            dv[idx, g] += dVp.numpy()
    return dq, dk, dv


# ---------------------------------------------------------------------------
# sampled forms (one output at a time; used at full workload sizes)


def forward_rows(q, k, v, topo, rows, scale=None, heads=None):
    """Forward for selected query tokens only, straight from V(i).

    Returns (out [n, Hq, D], lse [Hq, n]); heads outside ``heads`` are 0.
    """
    D = q.shape[2]
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(D, scale)
    heads = range(Hq) if heads is None else heads
    out = np.zeros((len(rows), Hq, D))
    lse = np.zeros((Hq, len(rows)))
    for r, i in enumerate(rows):
        vis = visible_tokens(topo, int(i))
        for g in sorted({h // G for h in heads}):
            K, V = _t(k[vis, g]), _t(v[vis, g])
            for h in [h for h in heads if h // G == g]:
                s = scale * (K @ _t(q[i, h]))
                m = s.max()
                e = torch.exp(s - m)
                out[r, h] = (e @ V / e.sum()).numpy()
                lse[h, r] = float(m + torch.log(e.sum()))
    return out, lse


def backward_rows(q, k, v, dout, topo, rows, scale=None):
    """dq for selected query tokens only (every head), straight from V(i)."""
    D = q.shape[2]
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(D, scale)
    out, lse = forward_rows(q, k, v, topo, rows, scale)
    dq = np.zeros((len(rows), Hq, D))
    for r, i in enumerate(rows):
        vis = visible_tokens(topo, int(i))
        for g in range(Hkv):
            K, V = _t(k[vis, g]), _t(v[vis, g])
            for h in range(g * G, (g + 1) * G):
                do = _t(dout[i, h])
                p = torch.exp(scale * (K @ _t(q[i, h])) - float(lse[h, r]))
                ds = p * (V @ do - do @ _t(out[r, h]))
                dq[r, h] = (scale * ds @ K).numpy()
    return dq


def backward_keys(q, k, v, dout, topo, keys, kv_head, scale=None):
    """dk, dv ([n, D] each) for selected key tokens of one key/value head.

    The queries that see key j are found from the definition: every token of
    a segment that has seg(j) as a strict ancestor, plus tokens i >= j of
    seg(j) itself.  Their lse/out come from the per-segment forward.
    """
    parent, st, ln = _arrays(topo)
    D = q.shape[2]
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(D, scale)
    seg_of = _segment_of_tokens(st, ln)
    hs = list(range(kv_head * G, (kv_head + 1) * G))
    tsegs = sorted({int(seg_of[j]) for j in keys})
    seers = {t: [u for u in range(len(parent)) if u == t or t in ancestors(parent, u)] for t in tsegs}
    needed = sorted({u for t in tsegs for u in seers[t]})
    out, lse = forward(q, k, v, topo, scale, heads=hs, segments=needed)
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for r, j in enumerate(keys):
        j = int(j)
        t = int(seg_of[j])
        qi = np.concatenate(
            [np.arange(j, st[t] + ln[t])] + [np.arange(st[u], st[u] + ln[u]) for u in seers[t] if u != t]
        )
        kj = _t(k[j, kv_head])
        vj = _t(v[j, kv_head])
        for h in hs:
            Q = _t(q[qi, h])
            dO = _t(dout[qi, h])
            p = torch.exp(scale * (Q @ kj) - _t(lse[h, qi]))
            delta = (dO * _t(out[qi, h])).sum(dim=1)
            ds = p * (dO @ vj - delta)
            dv[r] += (p @ dO).numpy()
            dk[r] += (scale * ds @ Q).numpy()
    return dk, dv


# ---------------------------------------------------------------------------
# brute force over a dense [T, T] mask (tiny inputs only)


def masked_dense_forward(q, k, v, topo, scale=None):
    """Same forward, as a dense masked softmax over all T keys."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    scale = _default_scale(D, scale)
    mask = visible_mask(topo)
    out = np.zeros_like(q)
    lse = np.zeros((Hq, T))
    for h in range(Hq):
        S = scale * q[:, h] @ k[:, h // G].T
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        out[:, h] = E @ v[:, h // G] / l
        lse[h] = (m + np.log(l))[:, 0]
    return out, lse


def masked_dense_backward(q, k, v, dout, topo, scale=None):
    """Same gradients from the dense masked form."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    scale = _default_scale(D, scale)
    mask = visible_mask(topo)
    out, lse = masked_dense_forward(q, k, v, topo, scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(Hq):
        g = h // G
        S = np.where(mask, scale * q[:, h] @ k[:, g].T, -np.inf)
        P = np.exp(S - lse[h][:, None])
        dv[:, g] += P.T @ dout[:, h]
        dP = dout[:, h] @ v[:, g].T
        delta = (dout[:, h] * out[:, h]).sum(axis=1, keepdims=True)
        dS = P * (dP - delta)
        dq[:, h] = scale * dS @ k[:, g]
        dk[:, g] += scale * dS.T @ q[:, h]
    return dq, dk, dv
