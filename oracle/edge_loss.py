"""Oracle for the sampled-edge projection and loss (test infrastructure
only: tests, the smoke check and the benchmark's CPU leg).

Megatron-LM pull request 7387 (section "Summary") picks out the hidden
states that are the source of a sampled edge before the vocabulary
projection; the issue "Shared-prefix training with context parallelism for
exact agent trajectories" (section "Describe the solution you'd like") sends
only those states through the vocabulary head and gives every sampled action
a single loss owner.  The pages name the loss no further; the reading taken here is the
plain next-token cross-entropy of each edge:

  logits[e] = W h[src[e]],   loss[e] = log sum_v exp(logits[e, v]) - logits[e, tgt[e]]

summed with weights dloss[e] by the caller, whose gradient is

  G[e, v] = (softmax(logits[e])_v - [v == tgt[e]]) dloss[e]
  dh[t]   = sum over edges e with src[e] = t of G[e] W      (rows of other tokens: 0)
  dW      = sum_e outer(G[e], h[src[e]]).

Everything is float64 NumPy, written straight from these definitions.

Parity pins (tests/test_edge_loss_oracle.py): W = 0 gives loss log V and a
closed-form dW; a two-word vocabulary gives log(1 + exp(other - target));
the log-sum-exp agrees with scipy's; adding one vector to every row of W
leaves the loss unchanged; dW sums to zero over the vocabulary; central
finite differences of the total loss match dh and dW; an edge repeated with
its weight split gives the same gradients.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def edge_logits(hidden, weight, src):
    """[E, V] logits of every edge: W h[src[e]]."""
    return _f64(hidden)[np.asarray(src, dtype=np.int64)] @ _f64(weight).T


def edge_loss_forward(hidden, weight, src, tgt):
    """(loss[E], lse[E]) of the sampled edges."""
    z = edge_logits(hidden, weight, src)
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    e = np.arange(z.shape[0])
    return lse - z[e, np.asarray(tgt, dtype=np.int64)], lse


def edge_loss_backward(hidden, weight, src, tgt, dloss):
    """(dh[T, d], dW[V, d]) of sum_e dloss[e] * loss[e]."""
    h, w = _f64(hidden), _f64(weight)
    src = np.asarray(src, dtype=np.int64)
    tgt = np.asarray(tgt, dtype=np.int64)
    z = h[src] @ w.T
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    p[np.arange(len(src)), tgt] -= 1.0
    g = p * _f64(dloss)[:, None]
    dh = np.zeros_like(h)
    np.add.at(dh, src, g @ w)
    dw = g.T @ h[src]
    return dh, dw
