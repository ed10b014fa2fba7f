"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Large workloads draw their inputs on the device (Philox,
seeded per head); the oracle receives host copies of exactly the sampled
heads' inputs and is compared on those heads' outputs and final states.

Workloads (q, k ~ N(0, 1/d), v ~ N(0, 1), bf16 inputs, fp32 state):
  * prefill B=1, H=8, N=4096, d=128, block 64      -- every head checked
  * prefill B=4, H=64, N=32768, d=128, block 128   -- 6 sampled heads
  * prefill B=1, H=64, N=1048576, d=128, block 128 -- heads 0, 21, 42, 63,
    with the value-column split and with the sequence split
  * one of 8 segments of that sequence, B=1, H=64, N=131072: the segment's
    K^T V (state accumulation) and its prefill from a non-zero initial state
    -- heads 0, 45
  * decode 256 x 64 heads, d=128, 128 steps, state = sum of 2048 outer
    products; fp32 state (gated) and bf16 state (drift reported)
"""
import os
import time

import numpy as np
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth
from oracle import oracle

from gpu_helpers import announce, dev, host, rel_err

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2


def _heads_to_host(t, heads):
    return np.stack([t[b, h].to(torch.float32).cpu().numpy() for b, h in heads])


def _check_sampled_prefill(B, H, N, d, block, cfg, heads, label, seqsplit=False):
    """The prefill on the whole workload, sampled heads against the oracle;
    with seqsplit, also lin_attn_prefill_seqsplit on the same inputs."""
    t0 = time.time()
    q, k, v = synth.prefill_inputs_device(cfg, B, H, N, d)
    o = torch.empty_like(q)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    announce(label, f"inputs ready in {time.time() - t0:.1f}s")
    la.prefill(q, k, v, o, S, block)
    torch.cuda.synchronize()
    outs = {"prefill": (np.stack([host(o[b, h]) for b, h in heads]), np.stack([host(S[b, h]) for b, h in heads]))}
    if seqsplit:
        assert la.prefill_seqsplit_workspace(B, H, N, d, block, torch.bfloat16) > 0
        S.zero_()
        la.prefill_seqsplit(q, k, v, o, S, block)
        torch.cuda.synchronize()
        outs["seqsplit"] = (np.stack([host(o[b, h]) for b, h in heads]),
                            np.stack([host(S[b, h]) for b, h in heads]))
    qh, kh, vh = (_heads_to_host(t, heads) for t in (q, k, v))
    del q, k, v, o
    torch.cuda.empty_cache()
    t1 = time.time()
    o_ref, S_ref = oracle.recurrence(qh, kh, vh)
    for name, (oh, Sh) in outs.items():
        eo, es = rel_err(oh, o_ref), rel_err(Sh, S_ref)
        print(f"  {label} {name}: heads {heads} rel err o={eo:.3e} state={es:.3e} (oracle {time.time() - t1:.1f}s)",
              flush=True)
        assert eo <= TOL_BF16 and es <= TOL_BF16, name


def test_workload_prefill_8x4096_all_heads():
    announce("workload prefill B1 H8 N4096 d128 blk64 (all heads)")
    B, H, N, d = 1, 8, 4096, 128
    q, k, v = synth.prefill_inputs(2, B, H, N, d)
    S0 = np.zeros((B, H, d, d), np.float32)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    od = torch.empty_like(qd)
    Sd = torch.zeros((B, H, d, d), device="cuda")
    la.prefill(qd, kd, vd, od, Sd, 64)
    torch.cuda.synchronize()
    eo, es = rel_err(host(od), o_ref), rel_err(host(Sd), S_ref)
    print(f"  chunked: rel err o={eo:.3e} state={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    # the token-by-token path on the same workload
    od2 = torch.empty_like(qd)
    Sd2 = torch.zeros((B, H, d, d), device="cuda")
    la.prefill_recurrent(qd, kd, vd, od2, Sd2)
    torch.cuda.synchronize()
    eo2, es2 = rel_err(host(od2), o_ref), rel_err(host(Sd2), S_ref)
    print(f"  recurrent: rel err o={eo2:.3e} state={es2:.3e}")
    assert eo2 <= TOL_BF16 and es2 <= 1e-4


def test_workload_prefill_4x64x32k_sampled():
    announce("workload prefill B4 H64 N32768 d128 blk128 (sampled heads)")
    _check_sampled_prefill(4, 64, 32768, 128, 128, 3,
                           [(0, 0), (0, 63), (1, 17), (2, 40), (3, 5), (3, 63)], "B4 H64 N32768")


def test_workload_prefill_1m_tokens_sampled():
    announce("workload prefill B1 H64 N1048576 d128 blk128 (heads 0,21,42,63)")
    _check_sampled_prefill(1, 64, 1 << 20, 128, 128, 4, [(0, 0), (0, 21), (0, 42), (0, 63)], "B1 H64 N1M",
                           seqsplit=True)


def test_workload_sequence_shard_sampled():
    announce("workload sequence shard B1 H64 N131072 d128 blk128 (heads 0,45)")
    B, H, N, d = 1, 64, 131072, 128
    heads = [(0, 0), (0, 45)]
    q, k, v = synth.prefill_inputs_device(6, B, H, N, d)
    dS = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    la.state_accumulate(k, v, dS)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator(device="cuda").manual_seed(6),
                     device="cuda", dtype=torch.float32)
    S = S0.clone()
    o = torch.empty_like(q)
    la.prefill(q, k, v, o, S, 128)
    torch.cuda.synchronize()
    qh, kh, vh = (_heads_to_host(t, heads) for t in (q, k, v))
    S0h = np.stack([host(S0[b, h]) for b, h in heads])
    dSh = np.stack([host(dS[b, h]) for b, h in heads])
    oh = np.stack([host(o[b, h]) for b, h in heads])
    Sh = np.stack([host(S[b, h]) for b, h in heads])
    del q, k, v, o
    torch.cuda.empty_cache()
    o_ref, S_ref = oracle.recurrence(qh, kh, vh, S0h)
    _, dS_ref = oracle.recurrence(np.zeros_like(kh), kh, vh)
    eo, es, ed = rel_err(oh, o_ref), rel_err(Sh, S_ref), rel_err(dSh, dS_ref)
    print(f"  shard: rel err o={eo:.3e} state={es:.3e} K^T V={ed:.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16 and ed <= TOL_BF16


def _decode_heads():
    return [((i * 37 + 3) % 256, (i * 11 + 5) % 64) for i in range(48)]


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_workload_decode_256x64_128_steps(state_dtype):
    announce("workload decode 256x64 d128, 128 steps, state", state_dtype)
    B, H, d, steps = 256, 64, 128, 128
    heads = _decode_heads()
    S0 = synth.decode_initial_state_device(B, H, d)
    S0_heads = np.stack([S0[b, h].cpu().numpy() for b, h in heads]).astype(np.float64)
    if state_dtype == "fp32":
        Sd = S0
    else:
        Sd = S0.to(torch.bfloat16)
        del S0
    S_true = S0_heads.copy()                              # fp64 truth from the fp32 S_0
    Sb_model = oracle.round_bf16_bits(S0_heads)           # bf16 storage model
    od = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    bi = torch.tensor([b for b, _ in heads], device="cuda")
    hi = torch.tensor([h for _, h in heads], device="cuda")
    worst_model, drift = 0.0, []
    for step in range(steps):
        q, k, v = synth.decode_step_inputs_device(step, B, H, d)
        la.decode(q, k, v, od, Sd)
        qh, kh, vh = (t[bi, hi].float().cpu().numpy() for t in (q, k, v))
        o_true = oracle.decode_step(qh, kh, vh, S_true)
        og = od[bi, hi].float().cpu().numpy().astype(np.float64)
        if state_dtype == "fp32":
            e = rel_err(og, o_true)
            worst_model = max(worst_model, e)
            assert e <= TOL_BF16, step
        else:
            o_model = oracle.decode_step_bf16_state(qh, kh, vh, Sb_model)
            worst_model = max(worst_model, rel_err(og, o_model))
            assert rel_err(og, o_model) <= TOL_BF16, step
            # continue the storage model from the kernel's stored state (see
            # the per-step ulp test in test_gpu_decode.py)
            Sb_model = Sd[bi, hi].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
            drift.append(rel_err(og, o_true))
    torch.cuda.synchronize()
    Sg = Sd[bi, hi].float().cpu().numpy().astype(np.float64)
    es = rel_err(Sg, S_true)
    if state_dtype == "fp32":
        print(f"  fp32 state: worst step rel err o={worst_model:.3e}, final state rel err={es:.3e}")
        assert es <= 1e-4
    else:
        print(f"  bf16 state: worst step rel err vs storage model={worst_model:.3e}; drift vs fp64 truth "
              f"o@1={drift[0]:.3e} o@32={drift[31]:.3e} o@128={drift[-1]:.3e} state@128={es:.3e}")
        assert np.isfinite(es)
