"""Seeded synthetic workloads for shared-prefix tree attention.

This module only *draws inputs*: segment topologies (parent, seg_start,
seg_len in DFS pre-order) and the q/k/v/dout tensors that go with them.  It
holds none of the attention arithmetic, so both the CPU oracle (``oracle/``)
and the GPU path can consume the same inputs without sharing any code.

Topologies follow the packed-sequence representation described in the
Megatron-LM issue "Shared-prefix training with context parallelism for exact
agent trajectories" (section "Describe the solution you'd like": DFS-linearized
segments with parent information) and the GRPO star/forest layout of the draft
"feat(hybrid): add opt-in shared-prefix attention and Mamba execution" (intro:
one prompt per packed group, each completion an independent suffix).  The
pages publish no dataset, so every workload here is synthetic.

Tensors are drawn chunk by chunk: chunk ``c`` (``CHUNK_TOKENS`` tokens) of
tensor ``name`` for seed ``s`` comes from
``numpy.random.default_rng([s, 1, TENSOR_IDS[name], c])`` as float32 standard
normals, scaled by the workload's std, then rounded to bfloat16 with
round-to-nearest-even (bf16 workloads) or kept as float32.  Chunk seeding makes
generation parallel and lets a caller regenerate any token range on its own.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Topology",
    "Workload",
    "WORKLOADS",
    "get_workload",
    "tiny_tree",
    "grpo_star",
    "agent_tree",
    "long_chain",
    "fragment_forest",
    "random_forest",
    "make_tensor",
    "bf16_to_f32",
    "f32_to_bf16",
    "CHUNK_TOKENS",
    "sampled_edges",
    "mamba_tensors",
]

CHUNK_TOKENS = 256
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "dout": 3, "hidden": 4, "weight": 5}


@dataclass
class Topology:
    """A DFS-linearized forest of token segments.

    parent[s] is -1 for a root, else the index of an earlier segment;
    segment s covers tokens [seg_start[s], seg_start[s] + seg_len[s]).
    ``source`` (optional) maps every physical token to the logical token it
    copies (used by fragment workloads, where ancestors are repeated).
    """

    parent: np.ndarray
    seg_start: np.ndarray
    seg_len: np.ndarray
    source: np.ndarray | None = None
    fragment_starts: list = field(default_factory=list)
    logical: "Topology | None" = None

    def __post_init__(self):
        self.parent = np.asarray(self.parent, dtype=np.int32)
        self.seg_start = np.asarray(self.seg_start, dtype=np.int32)
        self.seg_len = np.asarray(self.seg_len, dtype=np.int32)

    @property
    def num_segments(self) -> int:
        return int(self.parent.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.seg_start[-1] + self.seg_len[-1]) if self.num_segments else 0


def _from_dfs_list(nodes):
    """nodes: list of (parent_index, length) in DFS pre-order."""
    parent = np.array([p for p, _ in nodes], dtype=np.int32)
    seg_len = np.array([n for _, n in nodes], dtype=np.int32)
    seg_start = np.zeros_like(seg_len)
    if len(nodes) > 1:
        seg_start[1:] = np.cumsum(seg_len)[:-1]
    return Topology(parent, seg_start, seg_len)


def tiny_tree(root_len=64, child_len=32, children=4) -> Topology:
    """One root segment with ``children`` leaf branches (192 tokens by default)."""
    return _from_dfs_list([(-1, root_len)] + [(0, child_len)] * children)


def grpo_star(rng, groups=8, prompt_len=2048, completions=8, lo=256, hi=1024) -> Topology:
    """GRPO star forest: per group one prompt root and ``completions`` leaf
    children of length uniform{lo..hi}."""
    nodes = []
    for _ in range(groups):
        root = len(nodes)
        nodes.append((-1, prompt_len))
        for _ in range(completions):
            nodes.append((root, int(rng.integers(lo, hi + 1))))
    return _from_dfs_list(nodes)


def _log_uniform_len(rng, lo, hi):
    x = math.exp(rng.uniform(math.log(lo), math.log(hi)))
    return int(min(hi, max(lo, round(x))))


def _agent_tree_stream(rng, max_depth=6, lo=64, hi=4096, bmin=1, bmax=3):
    """Endless DFS pre-order stream of (depth, parent_offset_key, length).

    Yields (node_id, parent_id, length) with node ids counted from 0 across
    the whole stream; each tree has depth <= max_depth (root depth 0), a
    branching factor uniform{bmin..bmax} at every inner node and segment
    lengths log-uniform in [lo, hi].  Draw order per visited node: length,
    then (if depth < max_depth) the number of children.
    """
    node_id = 0
    while True:
        stack = [(-1, 0)]  # (parent id, depth)
        while stack:
            par, depth = stack.pop()
            length = _log_uniform_len(rng, lo, hi)
            me = node_id
            node_id += 1
            yield me, par, depth, length
            if depth < max_depth:
                nch = int(rng.integers(bmin, bmax + 1))
                for _ in range(nch):
                    stack.append((me, depth + 1))


def agent_tree(rng, total=65536, **kw) -> Topology:
    """Random agent-call tree truncated to ``total`` tokens in DFS order.

    If a tree is exhausted before ``total`` tokens, a new root starts (forest).
    The segment crossing ``total`` is cut so that T == total exactly.
    """
    nodes, ids, used = [], {}, 0
    for nid, par, _depth, length in _agent_tree_stream(rng, **kw):
        take = min(length, total - used)
        ids[nid] = len(nodes)
        nodes.append((ids[par] if par >= 0 else -1, take))
        used += take
        if used == total:
            break
    return _from_dfs_list(nodes)


def long_chain(rng, total=131072, trunk=40, every=5, side_lo=512, side_hi=2048) -> Topology:
    """Long strict-prefix chain: ``trunk`` trunk segments; after trunk segments
    every, 2*every, ... a side-leaf child of length uniform{side_lo..side_hi},
    visited before the trunk continues.  Trunk lengths split the remaining
    tokens evenly (remainder one token each on the first trunk segments)."""
    nside = trunk // every
    side = [int(rng.integers(side_lo, side_hi + 1)) for _ in range(nside)]
    rest = total - sum(side)
    base, rem = divmod(rest, trunk)
    trunk_len = [base + (1 if i < rem else 0) for i in range(trunk)]
    nodes, prev, si = [], -1, 0
    for i in range(trunk):
        me = len(nodes)
        nodes.append((prev, trunk_len[i]))
        if (i + 1) % every == 0:
            nodes.append((me, side[si]))
            si += 1
        prev = me
    return _from_dfs_list(nodes)


def fragment_forest(rng, fragments=4, capacity=32768, **kw) -> Topology:
    """Fragment-bounded forest: a stream of untruncated agent-call trees is
    packed in DFS order into ``fragments`` fragments of exactly ``capacity``
    tokens.  Every fragment is an independent forest: a fragment that starts
    inside a tree first holds copies of the next segment's ancestor chain
    (and, if that segment was split at the boundary, a copy of its already
    placed part, merged into the same segment), so each token still sees its
    whole ancestor path.  ``source`` maps physical tokens to logical tokens.
    """
    stream = _agent_tree_stream(rng, **kw)
    logical_parent, logical_start, logical_len = {}, {}, {}
    lpos = 0
    nodes, source = [], []
    frag_starts = []
    phys_of = {}  # logical id -> physical segment index in the current fragment
    used = 0  # tokens in current fragment
    frag = 0
    pending = None  # (logical id, tokens already placed)

    def chain(lid):
        out = []
        p = logical_parent[lid]
        while p >= 0:
            out.append(p)
            p = logical_parent[p]
        return out[::-1]

    def place(lid, lo, hi, phys_parent):
        nonlocal used
        nodes.append((phys_parent, hi - lo))
        source.extend(range(logical_start[lid] + lo, logical_start[lid] + hi))
        used += hi - lo
        return len(nodes) - 1

    while frag < fragments:
        if pending is None:
            nid, par, _d, length = next(stream)
            logical_parent[nid] = par
            logical_start[nid] = lpos
            logical_len[nid] = length
            lpos += length
            lid, done = nid, 0
        else:
            lid, done = pending
            pending = None
        if used == 0:
            frag_starts.append(len(nodes))
            phys_of = {}
            # repeat the ancestor chain so the fragment is self-contained
            for a in chain(lid):
                pp = phys_of.get(logical_parent[a], -1)
                phys_of[a] = place(a, 0, logical_len[a], pp)
        pp = phys_of.get(logical_parent[lid], -1)
        room = capacity - used
        # a split segment restarts with a copy of its already placed prefix
        lo = 0
        hi = min(logical_len[lid], lo + room)
        if done and hi < done:
            raise RuntimeError("ancestor chain does not fit a fragment")
        phys_of[lid] = place(lid, lo, hi, pp)
        if hi < logical_len[lid]:
            pending = (lid, hi)
        if used == capacity:
            frag += 1
            used = 0
    topo = _from_dfs_list(nodes)
    topo.source = np.asarray(source, dtype=np.int64)
    topo.fragment_starts = frag_starts
    # the unfragmented logical forest covering the same logical tokens
    n_logical = int(topo.source.max()) + 1
    lnodes = []
    for lid in sorted(logical_start):
        if logical_start[lid] >= n_logical:
            break
        take = min(logical_len[lid], n_logical - logical_start[lid])
        lnodes.append((logical_parent[lid], take))
    topo.logical = _from_dfs_list(lnodes)
    return topo


def comb(teeth, spine_len=2, leaf_len=1, tail_len=0) -> Topology:
    """A spine of ``teeth`` segments, each spine segment's first child a leaf
    of ``leaf_len`` tokens and its second the next spine segment.  In DFS
    order every spine segment is separated from its parent by that leaf, so
    the deepest spine segment's ancestor path splits into ``teeth`` separate
    token spans (``tail_len`` > 0 adds a last spine segment of that length,
    one more span)."""
    nodes = []
    parent = -1
    for _ in range(teeth):
        me = len(nodes)
        nodes.append((parent, spine_len))
        nodes.append((me, leaf_len))
        parent = me
    if tail_len:
        nodes.append((parent, tail_len))
    return _from_dfs_list(nodes)


def random_forest(rng, max_tokens=64, max_len=9, max_depth=4, p_new_root=0.15) -> Topology:
    """Small random DFS forest for brute-force tests: segment lengths
    uniform{1..max_len}, node depth <= max_depth, total <= max_tokens."""
    nodes, depth, used = [], [], 0
    path = []  # current root-to-last path (segment indices)
    while True:
        length = int(rng.integers(1, max_len + 1))
        if used + length > max_tokens:
            break
        if not path or rng.random() < p_new_root:
            par = -1
            path = []
        else:
            # attach to a random segment on the current path (keeps DFS order)
            cut = int(rng.integers(0, len(path)))
            while cut >= 0 and depth[path[cut]] >= max_depth:
                cut -= 1
            if cut < 0:
                par, path = -1, []
            else:
                par = path[cut]
                path = path[: cut + 1]
        me = len(nodes)
        nodes.append((par, length))
        depth.append(0 if par < 0 else depth[par] + 1)
        path.append(me)
        used += length
    if not nodes:
        nodes = [(-1, 1)]
    return _from_dfs_list(nodes)


def sampled_edges(topo: Topology, rng, vocab, p_sampled=0.5):
    """Sampled edges of a forest: (source token, sampled vocabulary id).

    Each segment is a sampled (model-generated) part with probability
    ``p_sampled``, else a prompt part.  Every token of a sampled segment is
    a sampled action, predicted from the token before it in its sequence:
    the previous token of the segment, or for the segment's first token the
    last token of its parent (a root's first token has no source and is not
    an edge).  A parent with several sampled children is thus the source of
    several edges.  Sampled ids are uniform over the vocabulary.  Returns
    int32 arrays (src, tgt), edges in token order."""
    src = []
    for s in range(topo.num_segments):
        if rng.random() >= p_sampled:
            continue
        a, n = int(topo.seg_start[s]), int(topo.seg_len[s])
        par = int(topo.parent[s])
        if par >= 0:
            src.append(int(topo.seg_start[par] + topo.seg_len[par] - 1))
        src.extend(range(a, a + n - 1))
    src = np.asarray(src, dtype=np.int32)
    tgt = rng.integers(0, vocab, size=src.size, dtype=np.int64).astype(np.int32)
    return src, tgt


def mamba_tensors(seed, tokens, heads=4, groups=2, head_dim=64, state_dim=128, channels=64, width=4):
    """float32 inputs of the Mamba path, drawn from one generator seeded with
    ``seed``, following a Mamba-2 mixer's initialisation ranges: x, B, C,
    conv input standard normal; dt log-uniform in [1e-3, 1e-1]; A = -U(1, 16);
    D standard normal; conv weight U(-1/sqrt(width), 1/sqrt(width)), bias
    U(-0.1, 0.1)."""
    rng = np.random.default_rng([seed, 7])
    f = np.float32
    out = {
        "x": rng.standard_normal((tokens, heads, head_dim), dtype=f),
        "dt": np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (tokens, heads))).astype(f),
        "A": (-rng.uniform(1.0, 16.0, heads)).astype(f),
        "B": rng.standard_normal((tokens, groups, state_dim), dtype=f),
        "C": rng.standard_normal((tokens, groups, state_dim), dtype=f),
        "D": rng.standard_normal(heads, dtype=f),
        "conv_x": rng.standard_normal((tokens, channels), dtype=f),
        "conv_w": rng.uniform(-1.0, 1.0, (channels, width)).astype(f) / f(np.sqrt(width)),
        "conv_b": rng.uniform(-0.1, 0.1, channels).astype(f),
    }
    return out


# ---------------------------------------------------------------------------
# tensors


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_chunk(out, name, seed, c, heads, dim, std, bf16, t_lo, t_hi):
    rng = np.random.default_rng([seed, 1, TENSOR_IDS[name], c])
    x = rng.standard_normal((CHUNK_TOKENS, heads, dim), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    lo = c * CHUNK_TOKENS
    a, b = max(lo, t_lo), min(lo + CHUNK_TOKENS, t_hi)
    part = x[a - lo : b - lo]
    out[a - t_lo : b - t_lo] = f32_to_bf16(part) if bf16 else part


def make_tensor(name, seed, tokens, heads, dim, std=1.0, dtype="bf16", t_lo=0, t_hi=None, threads=None):
    """Draw tensor ``name`` for tokens [t_lo, t_hi) of a [tokens, heads, dim]
    workload tensor.  bf16 tensors come back as uint16 bit patterns."""
    t_hi = tokens if t_hi is None else t_hi
    bf16 = dtype == "bf16"
    out = np.empty((t_hi - t_lo, heads, dim), dtype=np.uint16 if bf16 else np.float32)
    chunks = range(t_lo // CHUNK_TOKENS, (t_hi + CHUNK_TOKENS - 1) // CHUNK_TOKENS)
    threads = threads or min(16, os.cpu_count() or 1)
    if len(chunks) <= 2 or threads == 1:
        for c in chunks:
            _fill_chunk(out, name, seed, c, heads, dim, std, bf16, t_lo, t_hi)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda c: _fill_chunk(out, name, seed, c, heads, dim, std, bf16, t_lo, t_hi), chunks))
    return out


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload: topology recipe plus tensor shapes."""

    name: str
    kind: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "bf16" or "fp32"
    std: float
    backward: bool
    seed: int

    def topology(self) -> Topology:
        rng = np.random.default_rng([self.seed, 0])
        if self.kind == "tiny":
            return tiny_tree()
        if self.kind == "grpo_star":
            return grpo_star(rng)
        if self.kind == "agent_tree":
            return agent_tree(rng, total=65536)
        if self.kind == "long_chain":
            return long_chain(rng)
        if self.kind == "fragments":
            return fragment_forest(rng)
        raise ValueError(self.kind)

    def tensors(self, topo: Topology, names=("q", "k", "v", "dout"), t_lo=0, t_hi=None, threads=None):
        T = topo.total_tokens
        out = {}
        for n in names:
            h = self.num_kv_heads if n in ("k", "v") else self.num_q_heads
            out[n] = make_tensor(n, self.seed, T, h, self.head_dim, self.std, self.dtype, t_lo, t_hi, threads)
        return out


WORKLOADS = [
    Workload("tiny_tree_192_fp32", "tiny", 1, 1, 64, "fp32", 1.0, True, 1000),
    Workload("grpo_star_8x8_bf16", "grpo_star", 32, 8, 128, "bf16", 1.0, False, 1001),
    Workload("agent_tree_65536_bf16", "agent_tree", 32, 8, 128, "bf16", 1.0, True, 1002),
    Workload("long_chain_131072_bf16", "long_chain", 32, 8, 128, "bf16", 0.5, True, 1003),
    Workload("fragment_forest_4x32768_bf16", "fragments", 64, 8, 128, "bf16", 1.0, True, 1004),
]


def get_workload(key) -> Workload:
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS:
        if w.name == key:
            return w
    raise KeyError(key)
