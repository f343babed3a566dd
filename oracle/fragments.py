"""Oracle for bounded fragment planning with ancestor repetition (test
infrastructure only: tests, the smoke check and the benchmark's CPU leg).

Issue "Shared-prefix training with context parallelism for exact agent
trajectories", section "Describe the solution you'd like": fragments are
size-bounded, and ancestor segments may be duplicated in several of them
for that bound to hold.  The pages give the goal, not the steps; the reading
taken here (and by the library) is the plainest one that keeps attention
exact:

* walk the segments in DFS pre-order and fill fragments of at most
  ``max_tokens`` tokens in that order;
* a fragment that starts inside a tree first holds a copy of the ancestor
  chain of the segment it starts with (root first), so every token still
  sees its whole ancestor path;
* a segment that does not fit the rest of a fragment is split; the next
  fragment restarts it with a copy of the part already placed, in the same
  segment, so its tokens still see their causal prefix;
* copies are not loss owners; every source token is owned exactly once.

Parity pins (tests/test_fragments.py): every owned token's visible set,
mapped back to source tokens, equals its visible set in the source forest
(``tree_attention.visible_tokens``); ownership is exactly once; no fragment
exceeds the bound; each fragment is accepted as a DFS forest by the plan
builder; hand-worked small cases.
"""

from __future__ import annotations


def _children_order_ok(parent):
    return all(p < s for s, p in enumerate(parent) if p >= 0)


def fragment(parent, seg_start, seg_len, max_tokens):
    """Returns a list of fragments, each a dict of plain lists: parent,
    seg_len, source (source token per fragment token), owner (1/0)."""
    S = len(parent)
    assert _children_order_ok(parent)

    def chain_of(s):
        out = []
        a = parent[s]
        while a >= 0:
            out.append(a)
            a = parent[a]
        return list(reversed(out))

    # every root-to-leaf path must fit
    for s in range(S):
        if sum(seg_len[a] for a in chain_of(s)) + seg_len[s] > max_tokens:
            raise ValueError("a root-to-leaf path does not fit the bound")

    frags = []
    cur = None  # {"parent", "seg_len", "source", "owner", "where": {source seg: local index}}

    def new_fragment():
        return {"parent": [], "seg_len": [], "source": [], "owner": [], "where": {}}

    def used(fr):
        return len(fr["source"])

    def put(fr, s, n, copies):
        par = parent[s]
        fr["parent"].append(fr["where"][par] if par >= 0 else -1)
        fr["seg_len"].append(n)
        for o in range(n):
            fr["source"].append(seg_start[s] + o)
            fr["owner"].append(0 if o < copies else 1)
        fr["where"][s] = len(fr["seg_len"]) - 1

    for s in range(S):
        owned = 0
        while owned < seg_len[s]:
            if cur is None:
                cur = new_fragment()
                for a in chain_of(s):
                    put(cur, a, seg_len[a], seg_len[a])
            n = min(seg_len[s], max_tokens - used(cur))
            put(cur, s, n, owned)
            owned = n
            if used(cur) == max_tokens:
                frags.append(cur)
                cur = None
    if cur is not None:
        frags.append(cur)
    for fr in frags:
        del fr["where"]
    return frags
