"""Thin ctypes binding over ``lib/libtree_attn.so`` (the C ABI in
``include/tree_attn.h``).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is missing or a call fails, an exception is
raised.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libtree_attn.so")

OK = 0
INVALID_ARGUMENT = -1
UNSUPPORTED = -2
HIP_ERROR = -3
BF16 = 0
FP32 = 1

EXPORT_SPAN_PTR = 0
EXPORT_SPANS = 1
EXPORT_Q_TILES = 2
EXPORT_KV_TILES = 3
EXPORT_SEG_DEPTH = 4
EXPORT_SEG_PREFIX = 5
EXPORT_SEG_END = 6

# every symbol include/tree_attn.h declares
SYMBOLS = (
    "tree_attn_plan",
    "tree_attn_plan_query_run",
    "tree_attn_plan_query_run_host",
    "tree_attn_plan_host",
    "tree_attn_plan_async",
    "tree_attn_plan_destroy",
    "tree_attn_plan_info",
    "tree_attn_plan_export",
    "tree_attn_fwd",
    "tree_attn_fwd_workspace_bytes",
    "tree_attn_fwd_ws",
    "tree_attn_bwd_workspace_bytes",
    "tree_attn_bwd",
    "tree_attn_bwd_rowstat",
    "tree_attn_bwd_dkdv",
    "tree_attn_bwd_dq",
    "tree_attn_bwd_noalloc",
    "tree_attn_last_error",
    "tree_attn_fragment",
    "tree_attn_fragments_destroy",
    "tree_attn_fragments_info",
    "tree_attn_fragments_export",
    "tree_attn_edges",
    "tree_attn_edges_destroy",
    "tree_attn_edge_loss_workspace_bytes",
    "tree_attn_edge_loss_saved_bytes",
    "tree_attn_edge_loss_fwd",
    "tree_attn_edge_loss_bwd",
    "tree_attn_mamba_plan",
    "tree_attn_mamba_plan_host",
    "tree_attn_mamba_plan_destroy",
    "tree_attn_mamba_plan_info",
    "tree_attn_mamba_plan_export",
    "tree_attn_conv_fwd",
    "tree_attn_conv_bwd_workspace_bytes",
    "tree_attn_conv_bwd",
    "tree_attn_ssm_states_bytes",
    "tree_attn_ssm_workspace_bytes",
    "tree_attn_ssm_fwd",
    "tree_attn_ssm_bwd_workspace_bytes",
    "tree_attn_ssm_bwd",
)

FRAG_SEG_PTR = 0
FRAG_TOKEN_PTR = 1
FRAG_SEG_PARENT = 2
FRAG_SEG_LEN = 3
FRAG_TOKEN_SOURCE = 4
FRAG_TOKEN_OWNER = 5


class TreeAttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("num_roots", ctypes.c_int32),
        ("max_depth", ctypes.c_int32),
        ("max_path_len", ctypes.c_int64),
        ("pairs", ctypes.c_int64),
        ("num_spans", ctypes.c_int32),
        ("num_q_tiles", ctypes.c_int32),
        ("num_kv_tiles", ctypes.c_int32),
        ("on_device", ctypes.c_int32),
        ("q_begin", ctypes.c_int32),
        ("q_end", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class FragmentsInfo(ctypes.Structure):
    _fields_ = [
        ("num_fragments", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("source_tokens", ctypes.c_int64),
        ("fragment_tokens", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class MambaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("num_units", ctypes.c_int32),
        ("unit_tokens", ctypes.c_int32),
        ("max_depth", ctypes.c_int32),
        ("max_conv_width", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class SsmShape(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("state_dim", ctypes.c_int32),
    ]


MAMBA_EXPORT = {"prev": 0, "unit_start": 1, "unit_len": 2, "unit_pred": 3}

_lib = None


def library():
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m shared_prefix_tree_amd.build` "
            "(there is no fallback implementation)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    lib.tree_attn_plan.argtypes = [i32p, i32p, i32p, ctypes.c_int32, ctypes.POINTER(vp)]
    for name in ("tree_attn_plan_query_run", "tree_attn_plan_query_run_host"):
        getattr(lib, name).argtypes = [i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(vp)]
    lib.tree_attn_plan_host.argtypes = [i32p, i32p, i32p, ctypes.c_int32, ctypes.POINTER(vp)]
    lib.tree_attn_plan_async.argtypes = [i32p, i32p, i32p, ctypes.c_int32, vp, ctypes.POINTER(vp)]
    lib.tree_attn_plan_destroy.argtypes = [vp]
    lib.tree_attn_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.tree_attn_plan_export.argtypes = [vp, ctypes.c_int32, i32p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    lib.tree_attn_fwd.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Shape), vp, vp, vp]
    lib.tree_attn_fwd_workspace_bytes.argtypes = [vp, ctypes.POINTER(Shape)]
    lib.tree_attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tree_attn_fwd_ws.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Shape), vp, vp, vp, ctypes.c_size_t, vp]
    lib.tree_attn_bwd_workspace_bytes.argtypes = [vp, ctypes.POINTER(Shape)]
    lib.tree_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tree_attn_bwd.argtypes = [vp] * 6 + [vp, ctypes.POINTER(Shape)] + [vp] * 4 + [ctypes.c_size_t, vp]
    lib.tree_attn_bwd_rowstat.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Shape), vp, ctypes.c_size_t, vp]
    lib.tree_attn_bwd_dkdv.argtypes = [vp] * 6 + [ctypes.POINTER(Shape), vp, vp, vp, ctypes.c_size_t, vp]
    lib.tree_attn_bwd_dq.argtypes = [vp] * 6 + [ctypes.POINTER(Shape), vp, vp, ctypes.c_size_t, vp]
    lib.tree_attn_bwd_noalloc.argtypes = [vp] * 6 + [vp, ctypes.POINTER(Shape)] + [vp] * 4
    lib.tree_attn_last_error.restype = ctypes.c_char_p
    lib.tree_attn_fragment.argtypes = [i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(vp)]
    lib.tree_attn_fragments_destroy.argtypes = [vp]
    lib.tree_attn_fragments_info.argtypes = [vp, ctypes.POINTER(FragmentsInfo)]
    lib.tree_attn_fragments_export.argtypes = [vp, ctypes.c_int32, i32p, ctypes.c_int64,
                                               ctypes.POINTER(ctypes.c_int64)]
    for name in ("tree_attn_fragment", "tree_attn_fragments_destroy", "tree_attn_fragments_info",
                 "tree_attn_fragments_export"):
        getattr(lib, name).restype = ctypes.c_int
    lib.tree_attn_edges.argtypes = [i32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(vp)]
    lib.tree_attn_edges_destroy.argtypes = [vp]
    lib.tree_attn_edge_loss_workspace_bytes.argtypes = [vp, ctypes.c_int32]
    lib.tree_attn_edge_loss_workspace_bytes.restype = ctypes.c_size_t
    lib.tree_attn_edge_loss_saved_bytes.argtypes = [vp]
    lib.tree_attn_edge_loss_saved_bytes.restype = ctypes.c_size_t
    lib.tree_attn_edge_loss_fwd.argtypes = [vp, vp, ctypes.c_int32, vp, vp, vp, vp, ctypes.c_size_t, vp,
                                            ctypes.c_size_t, vp]
    lib.tree_attn_edge_loss_bwd.argtypes = [vp, vp, ctypes.c_int32, vp, vp, vp, ctypes.c_size_t, vp, vp, vp, vp,
                                            ctypes.c_size_t, vp]
    for name in ("tree_attn_edges", "tree_attn_edges_destroy", "tree_attn_edge_loss_fwd", "tree_attn_edge_loss_bwd"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("tree_attn_mamba_plan", "tree_attn_mamba_plan_host"):
        getattr(lib, name).argtypes = [i32p, i32p, i32p, ctypes.c_int32, ctypes.POINTER(vp)]
    lib.tree_attn_mamba_plan_destroy.argtypes = [vp]
    lib.tree_attn_mamba_plan_info.argtypes = [vp, ctypes.POINTER(MambaPlanInfo)]
    lib.tree_attn_mamba_plan_export.argtypes = [vp, ctypes.c_int32, i32p, ctypes.c_int64,
                                                ctypes.POINTER(ctypes.c_int64)]
    lib.tree_attn_conv_fwd.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    lib.tree_attn_conv_bwd_workspace_bytes.argtypes = [vp, ctypes.c_int32, ctypes.c_int32]
    lib.tree_attn_conv_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tree_attn_conv_bwd.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    for name in ("tree_attn_ssm_states_bytes", "tree_attn_ssm_workspace_bytes"):
        getattr(lib, name).argtypes = [vp, ctypes.POINTER(SsmShape)]
        getattr(lib, name).restype = ctypes.c_size_t
    lib.tree_attn_ssm_fwd.argtypes = [vp] * 7 + [ctypes.POINTER(SsmShape), vp, vp, ctypes.c_size_t, vp,
                                                 ctypes.c_size_t, vp]
    lib.tree_attn_ssm_bwd_workspace_bytes.argtypes = [vp, ctypes.POINTER(SsmShape)]
    lib.tree_attn_ssm_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tree_attn_ssm_bwd.argtypes = [vp] * 8 + [ctypes.POINTER(SsmShape), vp, ctypes.c_size_t] + [vp] * 7 + \
        [ctypes.c_size_t, vp]
    for name in ("tree_attn_mamba_plan", "tree_attn_mamba_plan_host", "tree_attn_mamba_plan_destroy",
                 "tree_attn_mamba_plan_info", "tree_attn_mamba_plan_export", "tree_attn_conv_fwd",
                 "tree_attn_conv_bwd", "tree_attn_ssm_fwd", "tree_attn_ssm_bwd"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("tree_attn_plan", "tree_attn_plan_query_run", "tree_attn_plan_query_run_host",
                 "tree_attn_plan_host", "tree_attn_plan_destroy",
                 "tree_attn_plan_info",
                 "tree_attn_plan_export", "tree_attn_fwd", "tree_attn_bwd", "tree_attn_bwd_rowstat",
                 "tree_attn_bwd_dkdv", "tree_attn_bwd_dq"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc):
    if rc != OK:
        raise TreeAttnError(rc, library().tree_attn_last_error().decode())


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class Plan:
    """A tree-attention plan (owned by the library).

    ``device=True`` uploads the tables to the current HIP device (call under
    ``torch.cuda.device(...)`` to choose it); ``device=False`` builds a
    host-only plan for inspection.  ``query_run=(q_begin, q_end)`` restricts
    the queries to those tokens (``tree_attn_plan_query_run[_host]``).
    ``stream`` (a torch stream, whole-token plans only): upload the tables
    with a copy ordered on that stream (``tree_attn_plan_async``) instead of
    a synchronous one.
    """

    def __init__(self, parent, seg_start, seg_len, device=True, query_run=None, stream=None):
        lib = library()
        self._handle = None
        p, pp = _i32(parent)
        s, sp = _i32(seg_start)
        n, np_ = _i32(seg_len)
        if not (len(p) == len(s) == len(n)):
            raise ValueError("parent, seg_start and seg_len must have the same length")
        h = ctypes.c_void_p()
        if query_run is not None:
            qb, qe = (int(x) for x in query_run)
            fn = lib.tree_attn_plan_query_run if device else lib.tree_attn_plan_query_run_host
            _check(fn(pp, sp, np_, ctypes.c_int32(len(p)), ctypes.c_int32(qb), ctypes.c_int32(qe), ctypes.byref(h)))
        elif stream is not None and device:
            _check(lib.tree_attn_plan_async(pp, sp, np_, ctypes.c_int32(len(p)), ctypes.c_void_p(stream.cuda_stream),
                                            ctypes.byref(h)))
        else:
            fn = lib.tree_attn_plan if device else lib.tree_attn_plan_host
            _check(fn(pp, sp, np_, ctypes.c_int32(len(p)), ctypes.byref(h)))
        self._handle = h
        self.device_index = None
        if device:
            import torch

            self.device_index = torch.cuda.current_device()

    @classmethod
    def from_topology(cls, topo, device=True, query_run=None, stream=None):
        return cls(topo.parent, topo.seg_start, topo.seg_len, device=device, query_run=query_run, stream=stream)

    @property
    def handle(self):
        return self._handle

    def info(self) -> dict:
        inf = PlanInfo()
        _check(library().tree_attn_plan_info(self._handle, ctypes.byref(inf)))
        return inf.as_dict()

    def export(self, which) -> np.ndarray:
        lib = library()
        cnt = ctypes.c_int64()
        _check(lib.tree_attn_plan_export(self._handle, which, None, 0, ctypes.byref(cnt)))
        buf = np.zeros(max(1, cnt.value), dtype=np.int32)
        _check(
            lib.tree_attn_plan_export(
                self._handle, which, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cnt.value, ctypes.byref(cnt)
            )
        )
        out = buf[: cnt.value]
        if which in (EXPORT_SPANS, EXPORT_Q_TILES, EXPORT_KV_TILES):
            out = out.reshape(-1, 4)
        return out

    def close(self):
        if self._handle is not None and _lib is not None:
            _lib.tree_attn_plan_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fragment(parent, seg_start, seg_len, max_tokens):
    """Bounded fragment planning (``tree_attn_fragment``).  Returns a list of
    fragments, each a dict: ``parent``, ``seg_start``, ``seg_len`` (a DFS
    forest starting at token 0), ``source`` (source token of each token) and
    ``owner`` (1 owned, 0 repeated), plus the info record."""
    lib = library()
    p, pp = _i32(parent)
    s, sp = _i32(seg_start)
    n, np_ = _i32(seg_len)
    h = ctypes.c_void_p()
    _check(lib.tree_attn_fragment(pp, sp, np_, ctypes.c_int32(len(p)), ctypes.c_int32(int(max_tokens)),
                                  ctypes.byref(h)))
    try:
        inf = FragmentsInfo()
        _check(lib.tree_attn_fragments_info(h, ctypes.byref(inf)))
        tables = {}
        for which in (FRAG_SEG_PTR, FRAG_TOKEN_PTR, FRAG_SEG_PARENT, FRAG_SEG_LEN, FRAG_TOKEN_SOURCE,
                      FRAG_TOKEN_OWNER):
            cnt = ctypes.c_int64()
            _check(lib.tree_attn_fragments_export(h, which, None, 0, ctypes.byref(cnt)))
            buf = np.zeros(max(1, cnt.value), dtype=np.int32)
            _check(lib.tree_attn_fragments_export(h, which, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                  cnt.value, ctypes.byref(cnt)))
            tables[which] = buf[: cnt.value]
    finally:
        lib.tree_attn_fragments_destroy(h)
    sptr, tptr = tables[FRAG_SEG_PTR], tables[FRAG_TOKEN_PTR]
    frags = []
    for f in range(inf.num_fragments):
        ln = tables[FRAG_SEG_LEN][sptr[f]:sptr[f + 1]]
        frags.append({
            "parent": tables[FRAG_SEG_PARENT][sptr[f]:sptr[f + 1]],
            "seg_start": np.concatenate([[0], np.cumsum(ln)[:-1]]).astype(np.int32),
            "seg_len": ln,
            "source": tables[FRAG_TOKEN_SOURCE][tptr[f]:tptr[f + 1]],
            "owner": tables[FRAG_TOKEN_OWNER][tptr[f]:tptr[f + 1]],
        })
    return frags, inf.as_dict()


class EdgePlan:
    """Sampled edges (source token, sampled vocabulary index), grouped by
    source and uploaded to the current device (``tree_attn_edges``)."""

    def __init__(self, edge_src, edge_tgt, num_tokens, vocab):
        lib = library()
        self._handle = None
        s, sp = _i32(edge_src)
        t, tp = _i32(edge_tgt)
        if len(s) != len(t):
            raise ValueError("edge_src and edge_tgt must have the same length")
        h = ctypes.c_void_p()
        _check(lib.tree_attn_edges(sp, tp, ctypes.c_int32(len(s)), ctypes.c_int32(int(num_tokens)),
                                   ctypes.c_int32(int(vocab)), ctypes.byref(h)))
        self._handle = h
        self.num_edges, self.num_tokens, self.vocab = len(s), int(num_tokens), int(vocab)

    @property
    def handle(self):
        return self._handle

    def workspace_bytes(self, hidden):
        return int(library().tree_attn_edge_loss_workspace_bytes(self._handle, int(hidden)))

    def saved_bytes(self):
        return int(library().tree_attn_edge_loss_saved_bytes(self._handle))

    def close(self):
        if self._handle is not None and _lib is not None:
            _lib.tree_attn_edges_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _edge_check(hidden, weight, edges):
    import torch

    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    T, d = hidden.shape
    if T != edges.num_tokens or tuple(weight.shape) != (edges.vocab, d):
        raise ValueError(f"expected hidden [{edges.num_tokens}, d] and weight [{edges.vocab}, d]")
    for name, t in (("hidden", hidden), ("weight", weight)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    return d


def edge_loss_fwd(hidden, weight, edges: EdgePlan, workspace=None, stream=None, saved=None):
    """Per-edge loss and log-sum-exp (``tree_attn_edge_loss_fwd``).  ``saved``:
    None, or a uint8 device buffer of ``edges.saved_bytes()`` that the
    forward fills with the logits for the backward."""
    import torch

    d = _edge_check(hidden, weight, edges)
    dev = hidden.device
    loss = torch.empty(edges.num_edges, dtype=torch.float32, device=dev)
    lse = torch.empty_like(loss)
    if workspace is None:
        workspace = torch.empty(max(256, edges.workspace_bytes(d)), dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        _check(library().tree_attn_edge_loss_fwd(hidden.data_ptr(), weight.data_ptr(), d, edges.handle,
                                                 loss.data_ptr(), lse.data_ptr(),
                                                 saved.data_ptr() if saved is not None else None,
                                                 saved.numel() if saved is not None else 0, workspace.data_ptr(),
                                                 workspace.numel(), ctypes.c_void_p(s.cuda_stream)))
    return loss, lse


def edge_loss_bwd(hidden, weight, edges: EdgePlan, lse, dloss, workspace=None, stream=None, saved=None):
    """Gradients (dhidden, dweight) of sum_e dloss[e] * loss[e]; ``saved``:
    the forward's saved logits, or None to recompute them."""
    import torch

    d = _edge_check(hidden, weight, edges)
    dev = hidden.device
    for name, t in (("lse", lse), ("dloss", dloss)):
        if t.dtype != torch.float32 or t.numel() != edges.num_edges or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of {edges.num_edges} elements")
    dh = torch.empty_like(hidden)
    dw = torch.empty_like(weight)
    if workspace is None:
        workspace = torch.empty(max(256, edges.workspace_bytes(d)), dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        _check(library().tree_attn_edge_loss_bwd(hidden.data_ptr(), weight.data_ptr(), d, edges.handle,
                                                 lse.data_ptr(), saved.data_ptr() if saved is not None else None,
                                                 saved.numel() if saved is not None else 0, dloss.data_ptr(),
                                                 dh.data_ptr(), dw.data_ptr(), workspace.data_ptr(),
                                                 workspace.numel(), ctypes.c_void_p(s.cuda_stream)))
    return dh, dw


class MambaPlan:
    """Tables of the Mamba path for one forest (``tree_attn_mamba_plan``):
    each token's predecessor, the convolution halo and the scan units.
    ``device=False`` builds a host-only plan for inspection."""

    def __init__(self, parent, seg_start, seg_len, device=True):
        lib = library()
        self._handle = None
        p, pp = _i32(parent)
        s, sp = _i32(seg_start)
        n, np_ = _i32(seg_len)
        if not (len(p) == len(s) == len(n)):
            raise ValueError("parent, seg_start and seg_len must have the same length")
        h = ctypes.c_void_p()
        fn = lib.tree_attn_mamba_plan if device else lib.tree_attn_mamba_plan_host
        _check(fn(pp, sp, np_, ctypes.c_int32(len(p)), ctypes.byref(h)))
        self._handle = h
        self.device = device
        self.num_tokens = int(self.info()["num_tokens"])

    @classmethod
    def from_topology(cls, topo, device=True):
        return cls(topo.parent, topo.seg_start, topo.seg_len, device=device)

    @property
    def handle(self):
        return self._handle

    def info(self) -> dict:
        info = MambaPlanInfo()
        _check(library().tree_attn_mamba_plan_info(self._handle, ctypes.byref(info)))
        return info.as_dict()

    def export(self, which):
        lib = library()
        code = MAMBA_EXPORT[which]
        count = ctypes.c_int64()
        _check(lib.tree_attn_mamba_plan_export(self._handle, code, None, 0, ctypes.byref(count)))
        buf = np.zeros(count.value, dtype=np.int32)
        _check(lib.tree_attn_mamba_plan_export(self._handle, code, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                               count.value, ctypes.byref(count)))
        return buf

    def close(self):
        if self._handle is not None and _lib is not None:
            _lib.tree_attn_mamba_plan_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _f32(name, t, shape=None):
    import torch

    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _plan_rows(name, t, plan):
    if t.shape[0] != plan.num_tokens:
        raise ValueError(f"{name} has {t.shape[0]} rows, the plan has {plan.num_tokens} tokens")


def _stream_of(t, stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def conv_fwd(x, weight, bias, plan: MambaPlan, out=None, stream=None):
    """Tree-causal depthwise convolution (``tree_attn_conv_fwd``):
    x [T, C], weight [C, W], bias [C] -> y [T, C]."""
    import torch

    T, C = x.shape
    W = weight.shape[1]
    _f32("x", x), _f32("weight", weight, (C, W)), _f32("bias", bias, (C,))
    _plan_rows("x", x, plan)
    y = out if out is not None else torch.empty_like(x)
    _f32("out", y, (T, C))
    with torch.cuda.device(x.device):
        _check(library().tree_attn_conv_fwd(x.data_ptr(), weight.data_ptr(), bias.data_ptr(), T, C, W, plan.handle,
                                            y.data_ptr(), _stream_of(x, stream)))
    return y


def conv_bwd(x, weight, dy, plan: MambaPlan, workspace=None, stream=None):
    """(dx, dweight, dbias) of sum <dy, y> (``tree_attn_conv_bwd``)."""
    import torch

    T, C = x.shape
    W = weight.shape[1]
    _f32("x", x), _f32("weight", weight, (C, W)), _f32("dy", dy, (T, C))
    _plan_rows("x", x, plan)
    dx, dw, db = torch.empty_like(x), torch.empty_like(weight), torch.empty(C, dtype=torch.float32, device=x.device)
    lib = library()
    if workspace is None:
        workspace = torch.empty(max(256, lib.tree_attn_conv_bwd_workspace_bytes(plan.handle, C, W)),
                                dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib.tree_attn_conv_bwd(x.data_ptr(), weight.data_ptr(), dy.data_ptr(), T, C, W, plan.handle,
                                      dx.data_ptr(), dw.data_ptr(), db.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), _stream_of(x, stream)))
    return dx, dw, db


def _ssm_shape(x, B):
    T, H, P = x.shape
    _, G, N = B.shape
    return SsmShape(T, H, P, G, N)


def ssm_states_bytes(plan: MambaPlan, num_heads, head_dim, num_groups, state_dim):
    sh = SsmShape(plan.info()["num_tokens"], num_heads, head_dim, num_groups, state_dim)
    return int(library().tree_attn_ssm_states_bytes(plan.handle, ctypes.byref(sh)))


def ssm_fwd(x, dt, A, B, C, D, plan: MambaPlan, out=None, states=None, workspace=None, stream=None):
    """State-space recurrence along the forest (``tree_attn_ssm_fwd``):
    returns y [T, H, P] and the saved states (uint8 device buffer) that the
    backward reads."""
    import torch

    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    for name, t, shp in (("x", x, None), ("dt", dt, (T, H)), ("A", A, (H,)), ("B", B, (T, G, N)),
                         ("C", C, (T, G, N)), ("D", D, (H,))):
        _f32(name, t, shp)
    _plan_rows("x", x, plan)
    sh = _ssm_shape(x, B)
    lib = library()
    y = out if out is not None else torch.empty_like(x)
    _f32("out", y, (T, H, P))
    nst = lib.tree_attn_ssm_states_bytes(plan.handle, ctypes.byref(sh))
    if states is None:
        states = torch.empty(max(256, nst), dtype=torch.uint8, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(256, lib.tree_attn_ssm_workspace_bytes(plan.handle, ctypes.byref(sh))),
                                dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib.tree_attn_ssm_fwd(x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(),
                                     D.data_ptr(), plan.handle, ctypes.byref(sh), y.data_ptr(), states.data_ptr(),
                                     states.numel(), workspace.data_ptr(), workspace.numel(),
                                     _stream_of(x, stream)))
    return y, states


def ssm_bwd(x, dt, A, B, C, D, dy, plan: MambaPlan, states, workspace=None, stream=None):
    """Gradients (dx, ddt, dA, dB, dC, dD) of sum <dy, y> (``tree_attn_ssm_bwd``);
    ``states`` is what ``ssm_fwd`` returned for the same inputs."""
    import torch

    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    for name, t, shp in (("x", x, None), ("dt", dt, (T, H)), ("A", A, (H,)), ("B", B, (T, G, N)),
                         ("C", C, (T, G, N)), ("D", D, (H,)), ("dy", dy, (T, H, P))):
        _f32(name, t, shp)
    _plan_rows("x", x, plan)
    sh = _ssm_shape(x, B)
    lib = library()
    if workspace is None:
        workspace = torch.empty(max(256, lib.tree_attn_ssm_bwd_workspace_bytes(plan.handle, ctypes.byref(sh))),
                                dtype=torch.uint8, device=x.device)
    dx, ddt, dA = torch.empty_like(x), torch.empty_like(dt), torch.empty_like(A)
    dB, dC, dD = torch.empty_like(B), torch.empty_like(C), torch.empty_like(D)
    with torch.cuda.device(x.device):
        _check(lib.tree_attn_ssm_bwd(x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(),
                                     D.data_ptr(), dy.data_ptr(), plan.handle, ctypes.byref(sh), states.data_ptr(),
                                     states.numel(), dx.data_ptr(), ddt.data_ptr(), dA.data_ptr(), dB.data_ptr(),
                                     dC.data_ptr(), dD.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                     _stream_of(x, stream)))
    return dx, ddt, dA, dB, dC, dD


def _shape(q, k, softmax_scale):
    import torch

    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q, k must be [T, H, D]")
    dt = {torch.bfloat16: BF16, torch.float32: FP32}.get(q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return Shape(q.shape[0], q.shape[1], k.shape[1], q.shape[2], dt, float(softmax_scale or 0.0))


def _check_tensor(name, t, like_dtype, shape, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != like_dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {like_dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(device, stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def tree_attn_fwd(q, k, v, plan: Plan, softmax_scale=0.0, out=None, lse=None, stream=None, workspace=None):
    """Forward pass.  q [T,Hq,D], k/v [T,Hkv,D] (bf16 or fp32, contiguous, on
    one GPU).  Returns (out [T,Hq,D], lse [Hq,T] float32).  With a device
    ``workspace`` (uint8, at least ``fwd_workspace_bytes``) the call is
    ``tree_attn_fwd_ws``: the same results, query tiles handed out through
    work-item counters."""
    import torch

    T, Hq, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _check_tensor("q", q, q.dtype, (T, Hq, D), dev)
    _check_tensor("k", k, q.dtype, (T, Hkv, D), dev)
    _check_tensor("v", v, q.dtype, (T, Hkv, D), dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    _check_tensor("out", out, q.dtype, (T, Hq, D), dev)
    _check_tensor("lse", lse, torch.float32, (Hq, T), dev)
    shape = _shape(q, k, softmax_scale)
    with torch.cuda.device(dev):
        if workspace is None:
            _check(library().tree_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), plan.handle,
                                           ctypes.byref(shape), out.data_ptr(), lse.data_ptr(),
                                           _stream_ptr(dev, stream)))
        else:
            _check(library().tree_attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), plan.handle,
                                              ctypes.byref(shape), out.data_ptr(), lse.data_ptr(),
                                              workspace.data_ptr(),
                                              ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                              _stream_ptr(dev, stream)))
    return out, lse


def fwd_workspace_bytes(plan: Plan, q, k, softmax_scale=0.0) -> int:
    shape = _shape(q, k, softmax_scale)
    return int(library().tree_attn_fwd_workspace_bytes(plan.handle, ctypes.byref(shape)))


def bwd_workspace_bytes(plan: Plan, q, k, softmax_scale=0.0) -> int:
    shape = _shape(q, k, softmax_scale)
    return int(library().tree_attn_bwd_workspace_bytes(plan.handle, ctypes.byref(shape)))


def tree_attn_bwd(q, k, v, out, lse, dout, plan: Plan, softmax_scale=0.0, dq=None, dk=None, dv=None,
                  workspace=None, stream=None):
    """Backward pass.  Returns (dq, dk, dv), each overwritten."""
    import torch

    T, Hq, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t, shp in (("q", q, (T, Hq, D)), ("k", k, (T, Hkv, D)), ("v", v, (T, Hkv, D)),
                         ("out", out, (T, Hq, D)), ("dout", dout, (T, Hq, D))):
        _check_tensor(name, t, q.dtype, shp, dev)
    _check_tensor("lse", lse, torch.float32, (Hq, T), dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, shp in (("dq", dq, (T, Hq, D)), ("dk", dk, (T, Hkv, D)), ("dv", dv, (T, Hkv, D))):
        _check_tensor(name, t, q.dtype, shp, dev)
    need = bwd_workspace_bytes(plan, q, k, softmax_scale)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    shape = _shape(q, k, softmax_scale)
    with torch.cuda.device(dev):
        _check(
            library().tree_attn_bwd(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                plan.handle, ctypes.byref(shape), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                workspace.data_ptr(), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                _stream_ptr(dev, stream),
            )
        )
    return dq, dk, dv


def tree_attn_bwd_noalloc(q, k, v, out, lse, dout, plan: Plan, dq, dk, dv, softmax_scale=0.0, stream=None):
    """Backward pass into caller-given dq, dk, dv with the library's fixed
    device scratch as workspace (``tree_attn_bwd_noalloc``): no device memory
    is allocated.  Calls that overlap on one GPU race."""
    import torch

    T, Hq, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t, shp in (("q", q, (T, Hq, D)), ("k", k, (T, Hkv, D)), ("v", v, (T, Hkv, D)),
                         ("out", out, (T, Hq, D)), ("dout", dout, (T, Hq, D)), ("dq", dq, (T, Hq, D)),
                         ("dk", dk, (T, Hkv, D)), ("dv", dv, (T, Hkv, D))):
        _check_tensor(name, t, q.dtype, shp, dev)
    _check_tensor("lse", lse, torch.float32, (Hq, T), dev)
    shape = _shape(q, k, softmax_scale)
    with torch.cuda.device(dev):
        _check(library().tree_attn_bwd_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            plan.handle, ctypes.byref(shape), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream_ptr(dev, stream)))
    return dq, dk, dv


def tree_attn_bwd_stages(q, k, v, out, lse, dout, plan: Plan, dq, dk, dv, workspace, softmax_scale=0.0,
                         stream=None, events=None):
    """Run the three backward stages as separate calls on one stream.

    Same result as ``tree_attn_bwd``.  ``events`` (optional): four
    ``torch.cuda.Event`` objects recorded before rowstat, dkdv, dq and after dq.
    """
    import torch

    lib = library()
    dev = q.device
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    for name, t, shp in (("q", q, (T, Hq, D)), ("k", k, (T, Hkv, D)), ("v", v, (T, Hkv, D)),
                         ("out", out, (T, Hq, D)), ("dout", dout, (T, Hq, D)), ("dq", dq, (T, Hq, D)),
                         ("dk", dk, (T, Hkv, D)), ("dv", dv, (T, Hkv, D))):
        _check_tensor(name, t, q.dtype, shp, dev)
    _check_tensor("lse", lse, torch.float32, (Hq, T), dev)
    shape = _shape(q, k, softmax_scale)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(s.cuda_stream)
    wsb = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    with torch.cuda.device(dev):
        if events:
            events[0].record(s)
        _check(lib.tree_attn_bwd_rowstat(out.data_ptr(), lse.data_ptr(), dout.data_ptr(), plan.handle,
                                         ctypes.byref(shape), workspace.data_ptr(), wsb, sp))
        if events:
            events[1].record(s)
        _check(lib.tree_attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                      plan.handle, ctypes.byref(shape), dk.data_ptr(), dv.data_ptr(),
                                      workspace.data_ptr(), wsb, sp))
        if events:
            events[2].record(s)
        _check(lib.tree_attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                    plan.handle, ctypes.byref(shape), dq.data_ptr(), workspace.data_ptr(), wsb, sp))
        if events:
            events[3].record(s)
    return dq, dk, dv
