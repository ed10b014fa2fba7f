"""GPU parity of the prefill with state snapshots (prefix cache): every
snapshot equals the oracle's state on that prefix, the outputs and final
state are bit-identical to the plain prefill's, and resuming from a snapshot
reproduces the rest of the sequence bit for bit."""
import numpy as np
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth
from oracle import oracle

from gpu_helpers import announce, dev, host, random_state, rel_err

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}


def run_snapshots(q, k, v, S0, block, every, dtype):
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    B, H, N, d = q.shape
    od = torch.empty_like(qd)
    Sd = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    ns = la.snapshot_count(N, block, every)
    snap = torch.full((B, H, ns, d, d), float("nan"), device="cuda")
    la.prefill_snapshots(qd, kd, vd, od, Sd, snap, block, every)
    # the plain prefill on the same inputs, for the bit-identity check
    od2 = torch.empty_like(qd)
    Sd2 = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    la.prefill(qd, kd, vd, od2, Sd2, block)
    torch.cuda.synchronize()
    assert torch.equal(od, od2) and torch.equal(Sd, Sd2)
    return host(od), host(Sd), host(snap)


def check_snapshots(q, k, v, S0, snap, block, every, tol, exact=False):
    ns = snap.shape[2]
    for s in range(ns):
        t = (s + 1) * every * block
        _, S_t = oracle.recurrence(q[:, :, :t], k[:, :, :t], v[:, :, :t], S0)
        if exact:
            np.testing.assert_array_equal(snap[:, :, s], S_t)
        else:
            e = rel_err(snap[:, :, s], S_t)
            assert e <= tol, (s, e)


@pytest.mark.parametrize("B,H,N,d,block,every,dtype", [
    (1, 2, 1000, 128, 128, 1, "bf16"), (1, 2, 1000, 128, 128, 3, "bf16"), (2, 3, 333, 64, 64, 2, "bf16"),
    (1, 2, 200, 128, 48, 1, "bf16"), (1, 2, 300, 64, 64, 1, "fp32"), (1, 1, 150, 128, 32, 2, "fp32"),
])
def test_snapshots_random(B, H, N, d, block, every, dtype):
    announce("prefill snapshots", B, H, N, d, block, every, dtype)
    q, k, v = synth.prefill_inputs(30, B, H, N, d, dtype)
    S0 = random_state(N, (B, H), d)
    o, S, snap = run_snapshots(q, k, v, S0, block, every, dtype)
    assert snap.shape[2] == (N // block) // every
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    assert rel_err(o, o_ref) <= TOL[dtype] and rel_err(S, S_ref) <= TOL[dtype]
    check_snapshots(q, k, v, S0, snap, block, every, TOL[dtype])


@pytest.mark.parametrize("d,block,N,every", [(128, 64, 300, 1), (64, 32, 200, 2)])
def test_snapshots_exact_integers(d, block, N, every):
    announce("prefill snapshots exact-integer", d, block, N, every)
    q, k, v = synth.integer_inputs(4000 + d + N, 1, 2, N, d)
    S0 = np.zeros((1, 2, d, d), np.float32)
    _, _, snap = run_snapshots(q, k, v, S0, block, every, "bf16")
    check_snapshots(q, k, v, S0, snap, block, every, 0.0, exact=True)


def test_resume_from_snapshot_is_bit_identical():
    """A later prefill of tokens t.. from snapshot S_t (t a block multiple)
    reproduces the full run's outputs and final state exactly."""
    announce("resume from snapshot")
    B, H, N, d, block, every = 1, 4, 900, 128, 128, 2
    q, k, v = synth.prefill_inputs(31, B, H, N, d, "bf16")
    S0 = random_state(3, (B, H), d)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    od = torch.empty_like(qd)
    Sd = torch.from_numpy(S0).cuda()
    snap = torch.empty((B, H, la.snapshot_count(N, block, every), d, d), device="cuda")
    la.prefill_snapshots(qd, kd, vd, od, Sd, snap, block, every, )
    for s in range(snap.shape[2]):
        t = (s + 1) * every * block
        Sr = snap[:, :, s].clone()
        orr = torch.empty_like(qd[:, :, t:].contiguous())
        la.prefill(qd[:, :, t:].contiguous(), kd[:, :, t:].contiguous(), vd[:, :, t:].contiguous(), orr, Sr, block)
        torch.cuda.synchronize()
        assert torch.equal(orr, od[:, :, t:]), s
        assert torch.equal(Sr, Sd), s
