"""Shared helpers for the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np


def announce(*parts):
    """Name the case before it touches the GPU, so a failure can be placed."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str):
    """Exact upload of float32 host values (already representable in dtype)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    num = float(np.max(np.abs(a - b))) if a.size else 0.0
    return num / den if den > 0 else num


def gpu_prefill(q, k, v, S0, block, dtype, split=0):
    """Run the HIP prefill on host inputs; returns (o, S) as float64 host arrays."""
    import torch
    import linear_attention_lightning_amd as la
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    od = torch.empty_like(qd)
    Sd = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    la.prefill(qd, kd, vd, od, Sd, block, split=split)
    torch.cuda.synchronize()
    return host(od), host(Sd)


def random_state(seed, lead, d, scale=1.0):
    rng = np.random.default_rng([7, seed])
    return (rng.standard_normal((*lead, d, d)) * scale).astype(np.float32)
