"""Oracle for Mamba state forking on a shared-prefix forest (test
infrastructure only: tests, the smoke check and the benchmark's CPU leg).

The draft "feat(hybrid): add opt-in shared-prefix attention and Mamba
execution" (intro) has the Mamba mixer share the prompt once, fork its
recurrent state into each branch, run the convolution halo per branch, and
accumulate the branches' gradients into the shared prefix; the issue
"Shared-prefix training with context parallelism for exact agent
trajectories" (section "Describe the solution you'd like") asks that the
convolution and recurrent state at branch points stay differentiable.  The
pages do not write the mixer out.  The reading taken here is the plainest
one: every token continues the sequence of its ancestor path, so a token's
predecessor ``prev(i)`` is the token before it in its segment, or for a
segment's first token the last token of the parent segment (-1 at a root),
and the two recurrent parts of a Mamba-2 mixer run along that relation:

* depthwise causal convolution of width W over channels c:
    y[i, c] = bias[c] + sum_{j<W} w[c, j] x[prev^(W-1-j)(i), c]   (x[-1] = 0)
* the selective state-space recurrence with a scalar decay per head
  (head h reads group g = h // (H / G) of B and C):
    a_i = exp(dt[i, h] A[h])
    S_i = a_i S_prev(i) + dt[i, h] x[i, h, :] outer B[i, g, :]      (S_-1 = 0)
    y[i, h, :] = S_i C[i, g, :] + D[h] x[i, h, :]

Backward is the exact gradient of sum <dy, y> with every token counted once;
a branch point's state and halo receive the sum over its branches.
Everything is float64 NumPy, token by token in DFS order.

Parity pins (tests/test_mamba_oracle.py): the recurrence equals its
quadratic (state-space dual) form, a sum over the visible ancestor tokens
computed by explicit loops; on every root-to-leaf sequence the tree results
equal a plain chain run and the convolution equals numpy.convolve; central
finite differences of the loss match every gradient; tree gradients equal
the sums over per-sequence copies with each token's dy given to one copy.
"""

from __future__ import annotations

import numpy as np


def previous_token(topo):
    """prev[i]: the token before i on its root-to-leaf path (-1 at a root)."""
    T = topo.total_tokens
    prev = np.arange(-1, T - 1, dtype=np.int64)
    for s in range(topo.num_segments):
        a = int(topo.seg_start[s])
        p = int(topo.parent[s])
        prev[a] = -1 if p < 0 else int(topo.seg_start[p] + topo.seg_len[p] - 1)
    return prev


def _ancestor_token(prev, i, k):
    for _ in range(k):
        if i < 0:
            return -1
        i = prev[i]
    return i


def conv_forward(x, w, bias, topo):
    """y[T, C] of the tree-causal depthwise convolution (x [T, C], w [C, W])."""
    x, w, bias = (np.asarray(a, np.float64) for a in (x, w, bias))
    prev = previous_token(topo)
    T, W = x.shape[0], w.shape[1]
    y = np.tile(bias, (T, 1))
    for i in range(T):
        for j in range(W):
            src = _ancestor_token(prev, i, W - 1 - j)
            if src >= 0:
                y[i] += w[:, j] * x[src]
    return y


def conv_backward(dy, x, w, topo):
    """(dx, dw, dbias) of sum <dy, y>."""
    dy, x, w = (np.asarray(a, np.float64) for a in (dy, x, w))
    prev = previous_token(topo)
    T, W = x.shape[0], w.shape[1]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for i in range(T):
        for j in range(W):
            src = _ancestor_token(prev, i, W - 1 - j)
            if src >= 0:
                dx[src] += w[:, j] * dy[i]
                dw[:, j] += dy[i] * x[src]
    return dx, dw, dy.sum(axis=0)


def _group_of(H, G):
    assert H % G == 0
    return np.arange(H) // (H // G)


def ssm_states(x, dt, A, B, topo):
    """All states S[T, H, P, N] of the tree recurrence."""
    x, dt, A, B = (np.asarray(a, np.float64) for a in (x, dt, A, B))
    T, H, P = x.shape
    g = _group_of(H, B.shape[1])
    prev = previous_token(topo)
    S = np.zeros((T, H, P, B.shape[2]))
    for i in range(T):
        a = np.exp(dt[i] * A)  # [H]
        inject = (dt[i][:, None] * x[i])[:, :, None] * B[i][g][:, None, :]
        S[i] = inject if prev[i] < 0 else a[:, None, None] * S[prev[i]] + inject
    return S


def ssm_forward(x, dt, A, B, C, D, topo):
    """y[T, H, P] of the tree state-space recurrence."""
    x, C, D = (np.asarray(a, np.float64) for a in (x, C, D))
    S = ssm_states(x, dt, A, B, topo)
    g = _group_of(x.shape[1], C.shape[1])
    return np.einsum("thpn,thn->thp", S, C[:, g]) + D[None, :, None] * x


def ssm_backward(dy, x, dt, A, B, C, D, topo):
    """(dx, ddt, dA, dB, dC, dD) of sum <dy, y>."""
    dy, x, dt, A, B, C, D = (np.asarray(a, np.float64) for a in (dy, x, dt, A, B, C, D))
    T, H, P = x.shape
    g = _group_of(H, B.shape[1])
    prev = previous_token(topo)
    S = ssm_states(x, dt, A, B, topo)
    dx, ddt = np.zeros_like(x), np.zeros_like(dt)
    dA, dD = np.zeros_like(A), np.zeros_like(D)
    dB, dC = np.zeros_like(B), np.zeros_like(C)
    incoming = {}  # token -> gradient of its state from its successors
    for i in range(T - 1, -1, -1):
        Bi, Ci = B[i][g], C[i][g]  # [H, N]
        dS = dy[i][:, :, None] * Ci[:, None, :]
        if i in incoming:
            dS = dS + incoming.pop(i)
        a = np.exp(dt[i] * A)
        Sp = S[prev[i]] if prev[i] >= 0 else np.zeros_like(S[i])
        dD += (dy[i] * x[i]).sum(axis=1)
        dSB = np.einsum("hpn,hn->hp", dS, Bi)
        dx[i] = D[:, None] * dy[i] + dt[i][:, None] * dSB
        inner = np.einsum("hpn,hpn->h", dS, Sp)
        ddt[i] = A * a * inner + (x[i] * dSB).sum(axis=1)
        dA += dt[i] * a * inner
        np.add.at(dB[i], g, dt[i][:, None] * np.einsum("hpn,hp->hn", dS, x[i]))
        np.add.at(dC[i], g, np.einsum("hpn,hp->hn", S[i], dy[i]))
        if prev[i] >= 0:
            incoming[prev[i]] = incoming.get(prev[i], 0.0) + a[:, None, None] * dS
    return dx, ddt, dA, dB, dC, dD
