"""Benchmark: tree-attention ancestor-path TFLOP/s (forward + backward) on one GPU.

One step = one pass of the whole path over one batch: plan (validate the
segment forest, derive spans and tiles, upload), forward, and the three
backward stages.  Inputs are generated once and are resident in HBM before
the timed region.  FLOPs are algorithmic: 4*D*Hq*pairs forward and
10*D*Hq*pairs backward, with pairs = sum over tokens of the visible-set size
(from the plan).

Prints one JSON line.  Default workload: the agent-call tree of 65,536 tokens
(32 query heads, 8 key/value heads, head_dim 128, bf16).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "tree-attention ancestor-path TFLOP/s fwd+bwd and % bf16 MFMA peak, 1 GPU"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ("kernel_common.hpp", "fwd.hip", "bwd.hip")


def kernel_source_hash():
    import hashlib

    csrc = os.path.join(ROOT, "shared_prefix_tree_amd", "csrc")
    blob = b"".join(open(os.path.join(csrc, f), "rb").read() for f in KERNEL_SOURCES)
    return hashlib.sha256(blob).hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when it was taken on different kernel sources."""
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    k = rec.get("workloads", {}).get(workload, {}).get(kernel)
    return k.get("bytes_per_launch") if k else None


def measured_sclk(workload, kernel):
    """Shader clock (GHz) the kernel ran at in the committed rocprofv3 counter
    run (GRBM_GUI_ACTIVE per XCD over the dispatch time), or None when it was
    taken on different kernel sources."""
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    k = rec.get("workloads", {}).get(workload, {}).get(kernel)
    return k.get("observed_sclk_ghz") if k else None


def mamba_scan_traffic():
    """HBM bytes of the Mamba scan kernels per step (one forward, one backward)
    from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE record, or None when it
    was taken on a different mamba_tree.hip."""
    import hashlib

    try:
        rec = json.load(open(PROFILE_TRAFFIC)).get("mamba_agent_tree_65536", {})
        src = open(os.path.join(ROOT, "shared_prefix_tree_amd", "csrc", "mamba_tree.hip"), "rb").read()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != hashlib.sha256(src).hexdigest()[:16]:
        return None
    return rec.get("scan_bytes_per_step")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, topo, arrs, kv_heads=1, pair_fraction=0.5, reps=3):
    """Time the float64 oracle (unchanged) on a bounded sample of the same
    workload: the first ``kv_heads`` key/value heads (with their query
    heads) and the query segments, in index order, that hold about
    ``pair_fraction`` of the pairs.  The forward and the backward call are
    timed separately, median of ``reps`` runs each; the oracle's backward
    call recomputes the forward it needs, so the backward time is the
    difference of the two medians.  Credited with the sample's algorithmic
    FLOPs (4 D and 10 D per pair and query head)."""
    import numpy as np

    import oracle
    from workloads import bf16_to_f32

    G = w.num_q_heads // w.num_kv_heads
    x = {k: (bf16_to_f32(v) if w.dtype == "bf16" else v) for k, v in arrs.items()}
    per_seg = oracle.segment_pairs(topo)
    total = sum(per_seg)
    segs, got = [], 0
    for u, p in enumerate(per_seg):
        if got >= pair_fraction * total:
            break
        segs.append(u)
        got += p
    heads = [h for g in range(kv_heads) for h in range(g * G, (g + 1) * G)]
    t_fwd, t_call = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.forward(x["q"], x["k"], x["v"], topo, heads=heads, segments=segs)
        t_fwd.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        oracle.backward(x["q"], x["k"], x["v"], x["dout"], topo, kv_heads=list(range(kv_heads)), segments=segs)
        t_call.append(time.perf_counter() - t0)
    f_s, c_s = float(np.median(t_fwd)), float(np.median(t_call))
    b_s = max(c_s - f_s, 1e-9)
    unit = w.head_dim * G * kv_heads * got
    try:
        import torch

        threads = torch.get_num_threads()
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    return {
        "value": 14.0 * unit / c_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"float64 oracle, key/value heads 0..{kv_heads - 1} ({kv_heads * G} of {w.num_q_heads} query "
        f"heads), query segments 0..{len(segs) - 1} of {topo.num_segments} ({got} of {total} pairs); forward "
        f"and backward call timed separately, median of {reps}; value = 14 D pairs / backward call (which "
        f"recomputes the forward)",
        "fwd_s": round(f_s, 3),
        "bwd_s": round(b_s, 3),
        "fwd_tflops": round(4.0 * unit / f_s / 1e12, 5),
        "bwd_tflops": round(10.0 * unit / b_s / 1e12, 5),
        "dtype": "f64",
        "cpu_model": _cpu_model(),
        "os_cpu_count": os.cpu_count(),
        "torch_threads": int(threads),
    }


def fragment_planner(args):
    """Host timing and token counts of bounded fragment planning (the pages
    report their tree before and after fragmentation in tokens)."""
    import numpy as np

    import shared_prefix_tree_amd as sp
    from workloads import agent_tree, get_workload

    B = args.fragment_bound
    forests = [(args.workload, get_workload(args.workload).topology())]
    forests.append(("agent_trees_4194304", agent_tree(np.random.default_rng([7, 0]), total=1 << 22)))
    rows = []
    for name, topo in forests:
        times = []
        for _ in range(max(3, args.steps // 4)):
            t0 = time.perf_counter()
            frags, info = sp.fragment(topo.parent, topo.seg_start, topo.seg_len, B)
            times.append(time.perf_counter() - t0)
        ms = 1e3 * float(np.median(times))
        T, F = info["source_tokens"], info["fragment_tokens"]
        rows.append({"forest": name, "tokens": int(T), "segments": int(topo.num_segments),
                     "fragments": int(info["num_fragments"]), "fragment_tokens": int(F),
                     "repeated_pct": round(100.0 * (F - T) / T, 3), "host_ms": round(ms, 3),
                     "mtokens_per_s": round(T / (ms * 1e-3) / 1e6, 2)})
        log(f"{name}: {T} tokens -> {F} in {info['num_fragments']} fragments of <= {B} "
            f"(+{100.0 * (F - T) / T:.2f} %), {ms:.2f} ms")
    print(json.dumps({"metric": "bounded fragment planning (host)", "max_tokens": B,
                      "binding_includes_table_export": True, "forests": rows}), flush=True)


def balanced_runs(topo, R):
    """R contiguous query runs of (nearly) equal pair counts: token i sees
    A(s) + (offset in s) + 1 keys."""
    import numpy as np

    parent, st, ln = (np.asarray(x, np.int64) for x in (topo.parent, topo.seg_start, topo.seg_len))
    prefix = np.zeros(len(ln), np.int64)
    for s in range(len(ln)):
        if parent[s] >= 0:
            prefix[s] = prefix[parent[s]] + ln[parent[s]]
    per_token = np.concatenate([prefix[s] + np.arange(1, ln[s] + 1) for s in range(len(ln))])
    cum = np.cumsum(per_token)
    cuts = [int(np.searchsorted(cum, cum[-1] * r / R)) + 1 for r in range(1, R)]
    edges = [0, *cuts, int(cum.size)]
    return list(zip(edges[:-1], edges[1:]))


def query_run_shares(args, sp, w, topo, t, out, lse, dq, dk, dv, ws, pairs):
    """Times each rank's share (forward + backward of one query run against
    every key) and checks that out / dq rows equal the whole plan's and that
    the dK / dV shares sum to its gradient.  One JSON line."""
    import numpy as np
    import torch

    R = args.query_runs
    runs = balanced_runs(topo, R)
    whole = sp.Plan.from_topology(topo)
    sp.tree_attn_fwd(t["q"], t["k"], t["v"], whole, out=out, lse=lse)
    sp.tree_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], whole, dq=dq, dk=dk, dv=dv, workspace=ws)
    out_r, lse_r, dq_r = torch.empty_like(out), torch.empty_like(lse), torch.empty_like(dq)
    dk_r, dv_r = torch.empty_like(dk), torch.empty_like(dv)
    sum_dk = torch.zeros(dk.shape, dtype=torch.float64, device=dk.device)
    sum_dv = torch.zeros_like(sum_dk)
    T, Hq, D = t["q"].shape
    ranks = []
    exact = True
    for qb, qe in runs:
        plan = sp.Plan.from_topology(topo, query_run=(qb, qe))
        rp = plan.info()["pairs"]

        def share(events=None):
            if events:
                events[0].record()
            sp.tree_attn_fwd(t["q"], t["k"], t["v"], plan, out=out_r, lse=lse_r)
            if events:
                events[1].record()
            sp.tree_attn_bwd(t["q"], t["k"], t["v"], out_r, lse_r, t["dout"], plan, dq=dq_r, dk=dk_r, dv=dv_r,
                             workspace=ws)
            if events:
                events[2].record()

        for _ in range(args.warmup):
            share()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            share(ev[i])
        torch.cuda.synchronize()
        f_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
        b_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
        exact &= bool(torch.equal(out_r[qb:qe], out[qb:qe]) and torch.equal(dq_r[qb:qe], dq[qb:qe])
                      and torch.equal(lse_r[:, qb:qe], lse[:, qb:qe]))
        sum_dk += dk_r.double()
        sum_dv += dv_r.double()
        flops = 14.0 * D * Hq * rp
        ranks.append({"run": [int(qb), int(qe)], "pairs": int(rp), "fwd_ms": round(f_ms, 4),
                      "bwd_ms": round(b_ms, 4), "tflops": round(flops / ((f_ms + b_ms) * 1e-3) / 1e12, 2)})
        log(f"rank run [{qb}, {qe}): pairs {rp}, fwd {f_ms:.3f} ms, bwd {b_ms:.3f} ms")

    def rel(a, b):
        return float(torch.linalg.vector_norm(a - b.double()) / torch.linalg.vector_norm(b.double()))

    slowest = max(r["fwd_ms"] + r["bwd_ms"] for r in ranks)
    print(json.dumps({
        "metric": "query-run shares (one context-parallel rank each), fwd+bwd",
        "workload": w.name, "ranks": R, "pairs": int(pairs), "dtype": w.dtype,
        "per_rank": ranks,
        "slowest_rank_ms": round(slowest, 4),
        "sum_of_ranks_ms": round(sum(r["fwd_ms"] + r["bwd_ms"] for r in ranks), 4),
        "out_lse_dq_rows_bitwise_equal_whole": exact,
        "dk_sum_rel_l2_vs_whole": rel(sum_dk, dk),
        "dv_sum_rel_l2_vs_whole": rel(sum_dv, dv),
    }), flush=True)


def edge_loss(args):
    """Times the sampled-edge projection and loss: the workload's forest,
    every segment sampled with probability 1/4 (each sampled token is an
    edge from the token before it), a 4096-wide hidden state and a
    131,072-word bf16 vocabulary head.  Algorithmic work: 2 E d V flops
    forward (the logits), 4 E d V backward (dh and dW); the backward's
    recomputation of the logits is not counted.  One JSON line."""
    import numpy as np
    import torch

    import shared_prefix_tree_amd as sp
    from workloads import get_workload, make_tensor, sampled_edges

    d, V = 4096, 131072
    w = get_workload(args.workload)
    topo = w.topology()
    T = topo.total_tokens
    src, tgt = sampled_edges(topo, np.random.default_rng([w.seed, 5]), V, 0.25)
    E = int(src.size)
    log(f"edge loss: T={T} E={E} d={d} V={V}: generating inputs")
    dev = "cuda:0"

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    h = dev_bf16(make_tensor("hidden", w.seed, T, 1, d)[:, 0])
    W = dev_bf16(make_tensor("weight", w.seed, V, 1, d, std=0.02)[:, 0])
    dloss = torch.full((E,), 1.0 / E, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        edges = sp.EdgePlan(src, tgt, T, V)
    ws = torch.empty(edges.workspace_bytes(d), dtype=torch.uint8, device=dev)
    saved = torch.empty(edges.saved_bytes(), dtype=torch.uint8, device=dev)  # fp16 logits, forward -> backward
    loss, lse = sp.edge_loss_fwd(h, W, edges, workspace=ws, saved=saved)
    for _ in range(args.warmup):
        loss, lse = sp.edge_loss_fwd(h, W, edges, workspace=ws, saved=saved)
        sp.edge_loss_bwd(h, W, edges, lse, dloss, workspace=ws, saved=saved)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        loss, lse = sp.edge_loss_fwd(h, W, edges, workspace=ws, saved=saved)
        ev[i][1].record()
        dh, dW = sp.edge_loss_bwd(h, W, edges, lse, dloss, workspace=ws, saved=saved)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps * 1e3
    f_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    fwd_f, bwd_f = 2.0 * E * d * V, 4.0 * E * d * V
    tf = (fwd_f + bwd_f) / ((f_ms + b_ms) * 1e-3) / 1e12
    mean_loss = float(loss.double().mean())
    log(f"edge loss: fwd {f_ms:.3f} ms, bwd {b_ms:.3f} ms, {tf:.1f} TFLOP/s, mean loss {mean_loss:.4f} "
        f"(log V = {np.log(V):.4f})")
    print(json.dumps({
        "metric": "sampled-edge projection + loss, fwd+bwd", "value": round(tf, 2), "unit": "TFLOP/s",
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name} edges", "tokens": T, "edges": E, "hidden": d, "vocab": V,
                   "saved_logits_gb": round(edges.saved_bytes() / 1e9, 3)},
        "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
        "fwd_tflops": round(fwd_f / (f_ms * 1e-3) / 1e12, 2), "bwd_tflops": round(bwd_f / (b_ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "mean_loss": round(mean_loss, 5),
    }), flush=True)


def mamba(args):
    """Times Mamba state forking on the workload's forest: a Mamba-2 mixer of
    a 4096-wide model (128 heads of 64, 8 groups, state 128; convolution of
    width 4 over the 10,240 x/B/C channels), all float32.  Algorithmic work
    per token and head: 5 P N flops forward (state update 3, output 2),
    11 P N backward (gradient update 3, dx, dB, dC and the decay term 2
    each); the convolution is counted by bytes (one read of every input,
    one write of every output).  One JSON line."""
    import numpy as np
    import torch

    import shared_prefix_tree_amd as sp
    from workloads import get_workload

    H, G, P, N, W = 128, 8, 64, 128, 4
    CH = H * P + 2 * G * N
    w = get_workload(args.workload)
    topo = w.topology()
    T = topo.total_tokens
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    def uniform(lo, hi, *shape):
        return lo + (hi - lo) * torch.rand(*shape, generator=gen, device=dev, dtype=torch.float32)

    x, B, C, dy = normal(T, H, P), normal(T, G, N), normal(T, G, N), normal(T, H, P)
    dt = torch.exp(uniform(float(np.log(1e-3)), float(np.log(1e-1)), T, H))
    A, D = -uniform(1.0, 16.0, H), normal(H)
    cx, cdy = normal(T, CH), normal(T, CH)
    cw, cb = uniform(-0.5, 0.5, CH, W), uniform(-0.1, 0.1, CH)
    with torch.cuda.device(dev):
        plan = sp.MambaPlan.from_topology(topo)
    info = plan.info()
    log(f"mamba: T={T} units={info['num_units']} H={H} G={G} P={P} N={N} conv channels={CH}")

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev else (lambda i: None)
        rec(0)
        sp.conv_fwd(cx, cw, cb, plan)
        rec(1)
        _, states = sp.ssm_fwd(x, dt, A, B, C, D, plan)
        rec(2)
        sp.conv_bwd(cx, cw, cdy, plan)
        rec(3)
        sp.ssm_bwd(x, dt, A, B, C, D, dy, plan, states)
        rec(4)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps * 1e3
    ms = [float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(4)]
    cf, sf, cbw, sbw = ms
    unit = T * H * P * N
    f_fwd, f_bwd = 5.0 * unit, 11.0 * unit
    scan_tf = (f_fwd + f_bwd) / ((sf + sbw) * 1e-3) / 1e12
    conv_gbs = (8.0 * T * CH) / (cf * 1e-3) / 1e9, (12.0 * T * CH) / (cbw * 1e-3) / 1e9
    log(f"mamba: conv fwd {cf:.3f} ms ({conv_gbs[0]:.0f} GB/s), scan fwd {sf:.3f} ms, conv bwd {cbw:.3f} ms "
        f"({conv_gbs[1]:.0f} GB/s), scan bwd {sbw:.3f} ms; scan {scan_tf:.2f} TFLOP/s")
    print(json.dumps({
        "metric": "Mamba state forking (tree convolution + state-space scan), fwd+bwd, scan TFLOP/s",
        "value": round(scan_tf, 3), "unit": "TFLOP/s", "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall, 4), "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name} forest, Mamba-2 mixer", "tokens": T, "units": info["num_units"],
                   "heads": H, "groups": G, "head_dim": P, "state_dim": N, "conv_channels": CH, "conv_width": W},
        "conv_fwd_ms": round(cf, 4), "ssm_fwd_ms": round(sf, 4), "conv_bwd_ms": round(cbw, 4),
        "ssm_bwd_ms": round(sbw, 4),
        "ssm_fwd_tflops": round(f_fwd / (sf * 1e-3) / 1e12, 3), "ssm_bwd_tflops": round(f_bwd / (sbw * 1e-3) / 1e12, 3),
        "conv_fwd_gbs": round(conv_gbs[0], 1), "conv_bwd_gbs": round(conv_gbs[1], 1),
        "roofline": {"bound": "alu", "achieved": round(scan_tf, 3), "peak": 157.3, "unit": "TFLOP/s",
                     "frac": round(scan_tf / 157.3, 4), "traffic": mamba_scan_traffic(),
                     "peak_basis": "published fp32 rate (matrix cores, and vector units with packed fp32); "
                                   "the scan's vector passes are built without packed fp32 instructions, which "
                                   "caps them at 78.6 = 256 CU x 4 SIMD x 16 lanes x 2 flops x 2.4 GHz"},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="agent_tree_65536_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fwd-entry", choices=("ws", "plain"), default="ws",
                    help="forward entry point timed: tree_attn_fwd_ws (work-item counters in a workspace, the "
                         "default) or tree_attn_fwd (one workgroup per query tile); the results are bitwise equal")
    ap.add_argument("--cpu-kv-heads", type=int, default=1)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes, --steps times (scales HBM counters)")
    ap.add_argument("--fragment-bound", type=int, default=0, metavar="B",
                    help="only time the host fragment planner on the workload's forest and on a stream of "
                         "agent-call trees, fragments of at most B tokens (prints its own JSON line)")
    ap.add_argument("--query-runs", type=int, default=0, metavar="R",
                    help="only time the shares of R context-parallel ranks: query runs of equal pairs, "
                         "each against every key (prints its own JSON line)")
    ap.add_argument("--edge-loss", action="store_true",
                    help="only time the sampled-edge projection and loss on the workload's forest "
                         "(prints its own JSON line)")
    ap.add_argument("--mamba", action="store_true",
                    help="only time Mamba state forking (tree convolution and state-space scan, forward and "
                         "backward) on the workload's forest (prints its own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(sharding is described in the design notes); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    if args.fragment_bound:
        fragment_planner(args)
        return

    import torch

    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": args.steps}), flush=True)
        return

    if args.edge_loss:
        edge_loss(args)
        return
    if args.mamba:
        mamba(args)
        return

    import shared_prefix_tree_amd as sp
    from workloads import get_workload

    w = get_workload(args.workload)
    topo = w.topology()
    names = ("q", "k", "v", "dout") if w.backward else ("q", "k", "v")
    log(f"workload {w.name}: generating inputs")
    arrs = w.tensors(topo, names=names)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def gpu(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    t = {k: gpu(v) for k, v in arrs.items()}
    T, Hq, D = t["q"].shape
    Hkv = t["k"].shape[1]
    out = torch.empty_like(t["q"])
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    if w.backward:
        dq = torch.empty_like(t["q"])
        dk = torch.empty_like(t["k"])
        dv = torch.empty_like(t["v"])
    probe = sp.Plan.from_topology(topo)
    info = probe.info()
    pairs = info["pairs"]
    ws = torch.empty(max(256, sp.bwd_workspace_bytes(probe, t["q"], t["k"])), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(256, sp.fwd_workspace_bytes(probe, t["q"], t["k"])), dtype=torch.uint8, device=dev)
    del probe

    stages = ["fwd", "rowstat", "dkdv", "dq"] if w.backward else ["fwd"]
    plan_host_s = []
    if args.query_runs:
        query_run_shares(args, sp, w, topo, t, out, lse, dq, dk, dv, ws, pairs)
        return

    stream = torch.cuda.current_stream()

    def step(events=None):
        # the plan's tables are uploaded by a copy ordered on the step's stream
        t0 = time.perf_counter()
        plan = sp.Plan.from_topology(topo, stream=stream)
        plan_host_s.append(time.perf_counter() - t0)
        if events:
            events[0].record()
        sp.tree_attn_fwd(t["q"], t["k"], t["v"], plan, out=out, lse=lse,
                         workspace=fws if args.fwd_entry == "ws" else None)
        if w.backward:
            sp.tree_attn_bwd_stages(t["q"], t["k"], t["v"], out, lse, t["dout"], plan, dq, dk, dv, ws,
                                    events=events[1:] if events else None)
        elif events:
            events[1].record()
        return plan

    # host work of the plan alone (validation and tile lists, no upload)
    build_s = []
    for _ in range(3):
        t0 = time.perf_counter()
        sp.Plan.from_topology(topo, device=False)
        build_s.append(time.perf_counter() - t0)
    log(f"T={T} S={topo.num_segments} Hq={Hq} Hkv={Hkv} D={D} pairs={pairs}; warmup {args.warmup}")
    warm = [step() for _ in range(args.warmup)]
    torch.cuda.synchronize()
    warm.clear()  # (plans are destroyed only once their kernels are done)
    plan_host_s.clear()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    keep = []
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        keep.append(step(ev[i]))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    keep.clear()
    ms_per_step = elapsed / args.steps * 1e3
    stage_ms = {s: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, s in enumerate(stages)}

    fwd_flops = 4.0 * D * Hq * pairs
    bwd_flops = 10.0 * D * Hq * pairs if w.backward else 0.0
    total = fwd_flops + bwd_flops
    value = total / (ms_per_step * 1e-3) / 1e12
    # algorithmic FLOPs credited to each kernel: forward 4D per pair; the
    # key-major pass does S, dP, dV, dK (8D); the query-major pass adds dQ (2D)
    credit = {"fwd": fwd_flops, "rowstat": 0.0, "dkdv": 8.0 * D * Hq * pairs, "dq": 2.0 * D * Hq * pairs}
    kernels = {}
    for s in stages:
        tf = credit[s] / (stage_ms[s] * 1e-3) / 1e12
        kernels[s] = {"ms": round(stage_ms[s], 4), "tflops": round(tf, 2),
                      "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    dom = max((s for s in stages if s != "rowstat"), key=lambda s: stage_ms[s])
    traffic = measured_traffic(w.name, dom)
    achieved = credit[dom] / (stage_ms[dom] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MATRIX_TFLOPS
    fwd_ms = stage_ms["fwd"]
    bwd_ms = sum(stage_ms[s] for s in stages[1:])
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "tokens": int(T),
            "segments": int(topo.num_segments),
            "q_heads": int(Hq),
            "kv_heads": int(Hkv),
            "head_dim": int(D),
            "pairs": int(pairs),
            "max_path_len": int(info["max_path_len"]),
            "step": "plan + fwd + bwd" if w.backward else "plan + fwd",
        },
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2) if w.backward else None,
        "kernel_tflops_fwd_bwd": round(total / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
        # the plan's host build alone, and the whole plan call inside a step
        # (build, pinned staging, device allocation, and a copy queued on the
        # step's stream: the host does not wait for the previous step's kernels)
        "plan_build_ms": round(1e3 * float(np.median(build_s)), 4),
        "plan_call_ms": round(1e3 * float(np.mean(plan_host_s)), 4),
        "kernels": kernels,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
    }
    sclk = measured_sclk(w.name, dom)
    if sclk:
        # the published peak assumes 2.4 GHz; the same fraction against the
        # clock rocprofv3 observed for this kernel
        result["roofline"]["observed_sclk_ghz"] = sclk
        result["roofline"]["frac_at_observed_sclk"] = round(achieved / (peak * sclk / 2.4), 4)
    if not args.no_cpu_baseline and w.backward:
        log("cpu baseline (float64 oracle, bounded sample)")
        result["cpu_baseline"] = cpu_baseline(w, topo, arrs, args.cpu_kv_heads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
