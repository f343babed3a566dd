"""Helpers shared by the GPU parity tests and the smoke check."""

from __future__ import annotations

import math
import sys
import time

import numpy as np

from workloads import bf16_to_f32

# tolerances: rel-L2 over the compared elements; lse max-abs
TOL = {
    "bf16": {"out": 1e-2, "dq": 2.5e-2, "dk": 2.5e-2, "dv": 2.5e-2, "lse": 1e-3},
    "fp32": {"out": 1e-5, "dq": 1e-5, "dk": 1e-5, "dv": 1e-5, "lse": 1e-5},
}


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_torch(arr, dtype, device):
    """Generator output (bf16 bit patterns as uint16, or float32) -> GPU tensor."""
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host(t):
    """GPU tensor -> float32/float64 numpy (bf16 widened exactly)."""
    import torch

    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def oracle_inputs(arrs, dtype):
    """Generator arrays -> float32 arrays holding exactly the same values."""
    return {k: (bf16_to_f32(v) if dtype == "bf16" else np.asarray(v, np.float32)) for k, v in arrs.items()}


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


# Where the exact result is (nearly) zero -- dq and dk of a token that sees
# only itself are exactly 0 -- a relative error divides rounding noise by ~0;
# such tensors are checked by max-abs error against these bounds instead.
ZERO_RMS = 1e-4
ABS_TOL = {"bf16": 1e-3, "fp32": 1e-5}


def tensor_error(name, got, ref, dtype):
    """(error, bound) for one output tensor: rel-L2 against TOL, or max-abs
    against ABS_TOL when the exact tensor is essentially zero; lse always
    max-abs."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if name == "lse":
        return float(np.abs(got - ref).max()), TOL[dtype]["lse"]
    if np.linalg.norm(ref.ravel()) <= ZERO_RMS * math.sqrt(max(ref.size, 1)):
        return float(np.abs(got - ref).max()), ABS_TOL[dtype]
    return rel_l2(got, ref), TOL[dtype][name]
