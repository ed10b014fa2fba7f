"""Seeded synthetic inputs for causal linear attention.

This module is the only code shared by the HIP path's callers (tests, bench)
and the fp64 oracle's callers.  It draws random numbers and rounds them to
the I/O dtype; it holds none of the attention arithmetic.

Distributions (the workloads' stated recipe): q, k ~ N(0, 1/d) and
v ~ N(0, 1), i.i.d., drawn in float32, scaled in float32, then rounded to the
I/O dtype (bf16: round to nearest even).  Every tensor is seeded per
(config, tensor, batch, head) so any single head can be regenerated alone.

Two interchangeable backends:

* host  -- numpy ``default_rng([2025, cfg, tensor, b, h])``; used for every
  CPU test and for device runs small enough to upload from the host;
* device -- torch's counter-based (Philox) generator on the GPU, seeded with
  a 63-bit digest of the same tuple; used for the large workloads, whose
  host generation would take minutes.  The values differ from the host
  backend's, so a run that uses it hands the oracle host copies of exactly
  the device tensors it drew.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os

import numpy as np

SEED_ROOT = 2025
TENSOR_ID = {"q": 0, "k": 1, "v": 2, "k_init": 3, "v_init": 4}
DECODE_CFG = 5          # config id used by the decode workload's seeds
DECODE_OUTER = 2048     # outer products summed into the decode initial state


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, min(n, 16))


def seed_digest(*key: int) -> int:
    """63-bit seed for torch generators, derived from the numpy seed tuple."""
    st = np.random.SeedSequence([SEED_ROOT, *key]).generate_state(2, np.uint32)
    return int((int(st[0]) << 32 | int(st[1])) & ((1 << 63) - 1))


def scale_for(tensor: str, d: int) -> float:
    return 1.0 / math.sqrt(d) if tensor in ("q", "k", "k_init") else 1.0


def round_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even) and return them as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def host_normals(key, shape, scale: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """float32 array of N(0, scale^2) draws from default_rng([2025, *key]),
    rounded to ``dtype`` ("bf16" or "fp32") and returned as float32."""
    x = np.random.default_rng([SEED_ROOT, *key]).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        x = round_bf16_f32(x)
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def prefill_inputs(cfg: int, B: int, H: int, N: int, d: int, dtype: str = "bf16"):
    """Host backend: (q, k, v) float32 arrays [B, H, N, d] holding values of
    ``dtype``, seeded per (cfg, tensor, b, h)."""
    out = {t: np.empty((B, H, N, d), dtype=np.float32) for t in ("q", "k", "v")}
    jobs = [(t, b, h) for t in ("q", "k", "v") for b in range(B) for h in range(H)]

    def one(job):
        t, b, h = job
        out[t][b, h] = host_normals((cfg, TENSOR_ID[t], b, h), (N, d), scale_for(t, d), dtype)

    if len(jobs) == 1 or N * d < 65536:
        for j in jobs:
            one(j)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, jobs))
    return out["q"], out["k"], out["v"]


def prefill_inputs_device(cfg: int, B: int, H: int, N: int, d: int, dtype: str = "bf16",
                          device: str = "cuda"):
    """Device backend: (q, k, v) torch tensors [B, H, N, d] of ``dtype`` on
    ``device``, each head drawn by a Philox generator seeded per
    (cfg, tensor, b, h)."""
    import torch
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    res = []
    for t in ("q", "k", "v"):
        x = torch.empty((B, H, N, d), dtype=tdt, device=device)
        g = torch.Generator(device=device)
        for b in range(B):
            for h in range(H):
                g.manual_seed(seed_digest(cfg, TENSOR_ID[t], b, h))
                z = torch.randn((N, d), generator=g, device=device, dtype=torch.float32)
                s = scale_for(t, d)
                if s != 1.0:
                    z.mul_(s)
                x[b, h].copy_(z)   # rounds to nearest even for bf16
                del z
        res.append(x)
    return tuple(res)


def decode_step_inputs(step: int, B: int, H: int, d: int, dtype: str = "bf16"):
    """Host backend: (q, k, v) float32 [B, H, d] for one decode step."""
    return tuple(host_normals((DECODE_CFG, TENSOR_ID[t], 1000 + step), (B, H, d), scale_for(t, d), dtype)
                 for t in ("q", "k", "v"))


def decode_step_inputs_device(step: int, B: int, H: int, d: int, dtype: str = "bf16",
                              device: str = "cuda"):
    """Device backend: (q, k, v) torch tensors [B, H, d] for one decode step."""
    import torch
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    g = torch.Generator(device=device)
    res = []
    for t in ("q", "k", "v"):
        g.manual_seed(seed_digest(DECODE_CFG, TENSOR_ID[t], 1000 + step))
        z = torch.randn((B, H, d), generator=g, device=device, dtype=torch.float32)
        s = scale_for(t, d)
        if s != 1.0:
            z.mul_(s)
        res.append(z.to(tdt))
    return tuple(res)


def decode_initial_state(B: int, H: int, d: int, n_outer: int = DECODE_OUTER,
                         dtype: str = "bf16") -> np.ndarray:
    """Host backend: float32 [B, H, d, d] initial state, the sum over
    ``n_outer`` random outer products k_m v_m^T (k ~ N(0, 1/d), v ~ N(0, 1),
    rounded to ``dtype``), summed in float64 and rounded once to float32."""
    S = np.empty((B, H, d, d), dtype=np.float32)
    for b in range(B):
        kk = host_normals((DECODE_CFG, TENSOR_ID["k_init"], b), (H, n_outer, d), scale_for("k", d), dtype)
        vv = host_normals((DECODE_CFG, TENSOR_ID["v_init"], b), (H, n_outer, d), 1.0, dtype)
        S[b] = np.matmul(kk.astype(np.float64).transpose(0, 2, 1), vv.astype(np.float64)).astype(np.float32)
    return S


def decode_initial_state_device(B: int, H: int, d: int, n_outer: int = DECODE_OUTER,
                                dtype: str = "bf16", device: str = "cuda"):
    """Device backend of :func:`decode_initial_state` (float32 tensor on the GPU)."""
    import torch
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=device)
    g = torch.Generator(device=device)
    for b in range(B):
        g.manual_seed(seed_digest(DECODE_CFG, TENSOR_ID["k_init"], b))
        kk = torch.randn((H, n_outer, d), generator=g, device=device, dtype=torch.float32)
        kk.mul_(scale_for("k", d))
        g.manual_seed(seed_digest(DECODE_CFG, TENSOR_ID["v_init"], b))
        vv = torch.randn((H, n_outer, d), generator=g, device=device, dtype=torch.float32)
        kt = kk.to(tdt).to(torch.float64).transpose(1, 2).contiguous()
        vd = vv.to(tdt).to(torch.float64).contiguous()
        S[b].copy_(torch.bmm(kt, vd))
        del kk, vv, kt, vd
    return S


def integer_inputs(seed: int, B: int, H: int, N: int, d: int, max_nnz: int = 2):
    """Exact-integer inputs: each q, k, v row holds at most ``max_nnz``
    entries from {-1, +1}, the rest zeros.  Returns float32 [B, H, N, d]."""
    rng = np.random.default_rng([SEED_ROOT, 99, seed, B, H, N, d])
    out = []
    for _ in range(3):
        x = np.zeros((B, H, N, d), dtype=np.float32)
        nnz = rng.integers(0, max_nnz + 1, size=(B, H, N))
        for idx in np.ndindex(B, H, N):
            cols = rng.choice(d, size=int(nnz[idx]), replace=False)
            x[idx][cols] = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=len(cols))
        out.append(x)
    return tuple(out)
