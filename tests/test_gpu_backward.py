"""GPU parity of the backward pass (``lin_attn_backward``) against the fp64
oracle's gradients.

For L = sum_t <o_t, dO_t> + <S_N, dS_N> the kernel returns dq, dk, dv (bf16)
and dS_0 (fp32) from the chunked kernel in other roles: dQ as the forward
prefill of (dO, V, K) from S_0^T, dV and dK as prefills over the reversed
token order of (K, Q, dO) from dS_N and (V, dO, Q) from dS_N^T -- run as
separate passes, as one paired launch, or fused in one sweep
(``lin_attn_backward_ex``); every strategy is checked.

Gates: max|gpu - oracle| / max|oracle| <= 1e-2 for each of dq, dk, dv, dS_0
(bf16 inputs and outputs, fp32 accumulation and carried states, the gate of
the bf16 forward path), <= 1e-4 with fp32 inputs and outputs (the fp32
kernel in the same roles); bitwise for exact-integer inputs.
"""
import numpy as np
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth
from oracle import oracle

from gpu_helpers import announce, dev, host, random_state, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2


STRATEGIES = {"separate": la.BWD_SEPARATE, "paired": la.BWD_PAIRED, "fused": la.BWD_FUSED}


def gpu_backward(q, k, v, dO, S0, dSN, block, want_dS0=True, strategy=la.BWD_AUTO, dtype="bf16"):
    qd, kd, vd, dod = (dev(x, dtype) for x in (q, k, v, dO))
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    B, H, N, d = q.shape
    s0 = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, np.float32)).cuda()
    ds = None if dSN is None else torch.from_numpy(np.ascontiguousarray(dSN, np.float32)).cuda()
    ds0 = torch.full((B, H, d, d), float("nan"), device="cuda") if want_dS0 else None
    la.backward(qd, kd, vd, dod, dq, dk, dv, block, state0=s0, dstate=ds, dstate0=ds0, strategy=strategy)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), (host(ds0) if want_dS0 else None)


def grad_inputs(seed, B, H, N, d):
    q, k, v = synth.prefill_inputs(seed, B, H, N, d, "bf16")
    dO = synth.prefill_inputs(seed + 1000, B, H, N, d, "bf16")[2]  # N(0, 1) upstream gradients
    return q, k, v, dO


@pytest.mark.parametrize("strategy", sorted(STRATEGIES))
@pytest.mark.parametrize("B,H,N,d,block", [
    (1, 2, 1000, 128, 128), (2, 3, 333, 128, 64), (1, 2, 77, 128, 16), (1, 4, 517, 64, 96),
    (2, 2, 130, 64, 32), (1, 2, 1, 128, 64), (1, 130, 257, 128, 128), (1, 3, 700, 64, 128),
])
def test_backward_random(B, H, N, d, block, strategy):
    announce("backward random", B, H, N, d, block, strategy)
    q, k, v, dO = grad_inputs(60 + N, B, H, N, d)
    S0 = random_state(N, (B, H), d)
    dSN = random_state(N + 1, (B, H), d)
    ref = oracle.backward(q, k, v, dO, S0, dSN)
    got = gpu_backward(q, k, v, dO, S0, dSN, block, strategy=STRATEGIES[strategy])
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    print("  rel err dq={:.2e} dk={:.2e} dv={:.2e} dS0={:.2e}".format(*errs))
    assert max(errs) <= TOL, errs


@pytest.mark.parametrize("strategy", sorted(STRATEGIES))
@pytest.mark.parametrize("d,N,block", [(128, 300, 128), (128, 77, 32), (64, 129, 64)])
def test_backward_exact_integers(d, N, block, strategy):
    """Sparse {-1, 0, 1} inputs and small integer states: every product and
    partial sum is an integer within bf16's exact range, so the gradients
    are bitwise those of the oracle."""
    announce("backward exact integers", d, N, block)
    B, H = 1, 3
    q, k, v = synth.integer_inputs(900 + d + N, B, H, N, d)
    dO, _, _ = synth.integer_inputs(950 + d + N, B, H, N, d)
    rng = np.random.default_rng([61, d, N])
    S0 = rng.integers(-2, 3, (B, H, d, d)).astype(np.float64)
    dSN = rng.integers(-2, 3, (B, H, d, d)).astype(np.float64)
    ref = oracle.backward(q, k, v, dO, S0, dSN)
    for r in ref:
        assert np.abs(r).max() <= 256, "integer case leaves bf16's exact range"
    # the carried states stay in range too
    assert (np.abs(S0) + np.einsum("bhti,bhtj->bhij", np.abs(k), np.abs(v))).max() <= 256
    assert (np.abs(dSN) + np.einsum("bhti,bhtj->bhij", np.abs(q), np.abs(dO))).max() <= 256
    got = gpu_backward(q, k, v, dO, S0, dSN, block, strategy=STRATEGIES[strategy])
    for name, g, r in zip(("dq", "dk", "dv", "dS0"), got, ref):
        np.testing.assert_array_equal(g, r, err_msg=name)


def test_backward_null_states_and_no_tokens():
    """S_0 and dS_N may be NULL (zero); with N = 0 the gradient of S_0 is
    dS_N (or zero), and no token gradient is touched."""
    announce("backward null states / N = 0")
    B, H, N, d = 1, 3, 200, 128
    q, k, v, dO = grad_inputs(70, B, H, N, d)
    ref = oracle.backward(q, k, v, dO, None, None)
    got = gpu_backward(q, k, v, dO, None, None, 64)
    assert max(rel_err(g, r) for g, r in zip(got, ref)) <= TOL
    dSN = random_state(3, (B, H), d)
    e = np.zeros((B, H, 0, d), np.float32)
    for ds in (dSN, None):
        _, _, _, dS0 = gpu_backward(e, e, e, e, None, ds, 64)
        np.testing.assert_array_equal(dS0, np.zeros_like(dSN) if ds is None else dSN.astype(np.float64))


def test_backward_deterministic_and_consistent_with_forward():
    """Repeated calls are bitwise identical; the gradient of S_0 equals
    dS_N + Q^T dO, which the state accumulation computes independently."""
    announce("backward determinism")
    B, H, N, d = 1, 4, 700, 128
    q, k, v, dO = grad_inputs(71, B, H, N, d)
    S0 = random_state(5, (B, H), d)
    dSN = random_state(6, (B, H), d)
    runs = [gpu_backward(q, k, v, dO, S0, dSN, 128) for _ in range(2)]
    for a, b in zip(*runs):
        np.testing.assert_array_equal(a, b)
    qd, dod = dev(q, "bf16"), dev(dO, "bf16")
    acc = torch.from_numpy(dSN).cuda()
    la.state_accumulate(qd, dod, acc)
    torch.cuda.synchronize()
    assert rel_err(runs[0][3], host(acc)) <= 1e-5


def test_backward_workload_4x64x32k_sampled():
    """The headline prefill shape: gradients of all 256 sequences on the GPU,
    two heads checked against the oracle at full length."""
    announce("backward workload B=4 H=64 N=32768 sampled")
    B, H, N, d = 4, 64, 32768, 128
    q, k, v = synth.prefill_inputs_device(13, B, H, N, d)
    dO = synth.prefill_inputs_device(14, B, H, N, d)[2]
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ds0 = torch.empty((B, H, d, d), device="cuda")
    la.backward(q, k, v, dO, dq, dk, dv, 128, dstate0=ds0)
    torch.cuda.synchronize()
    for b, h in ((0, 5), (3, 60)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.backward(host(q[sl]), host(k[sl]), host(v[sl]), host(dO[sl]))
        got = (host(dq[sl]), host(dk[sl]), host(dv[sl]), host(ds0[sl]))
        errs = [rel_err(g, r) for g, r in zip(got, ref)]
        print(f"  head ({b}, {h}) rel err dq={errs[0]:.2e} dk={errs[1]:.2e} dv={errs[2]:.2e} dS0={errs[3]:.2e}")
        assert max(errs) <= TOL, errs


@pytest.mark.parametrize("d,block", [(128, 128), (64, 64), (128, 96)])
def test_backward_strategies_bitwise_equal(d, block):
    """The separate, paired and fused strategies compute the same products in
    the same order (the fused dK role reads the carried state's bf16 copy
    transposed, which holds the same values as the separate pass's own copy):
    their gradients agree bitwise, and the default picks one of them."""
    announce("backward strategies bitwise", d, block)
    B, H, N = 2, 3, 611
    q, k, v, dO = grad_inputs(72 + d, B, H, N, d)
    S0 = random_state(7, (B, H), d)
    dSN = random_state(8, (B, H), d)
    runs = {name: gpu_backward(q, k, v, dO, S0, dSN, block, strategy=code) for name, code in STRATEGIES.items()}
    runs["auto"] = gpu_backward(q, k, v, dO, S0, dSN, block)
    for name, got in runs.items():
        for gname, g, r in zip(("dq", "dk", "dv", "dS0"), got, runs["separate"]):
            np.testing.assert_array_equal(g, r, err_msg=f"{name} {gname}")


def test_backward_workload_4x64x32k_fused_vs_separate():
    """At the headline shape the default runs the fused sweep: every
    gradient equals the separate passes' bitwise."""
    announce("backward workload B=4 H=64 N=32768 fused vs separate")
    B, H, N, d = 4, 64, 32768, 128
    q, k, v = synth.prefill_inputs_device(13, B, H, N, d)
    dO = synth.prefill_inputs_device(14, B, H, N, d)[2]
    outs = {}
    for name in ("separate", "fused"):
        g = [torch.empty_like(q) for _ in range(3)] + [torch.empty((B, H, d, d), device="cuda")]
        la.backward(q, k, v, dO, g[0], g[1], g[2], 128, dstate0=g[3], strategy=STRATEGIES[name])
        torch.cuda.synchronize()
        outs[name] = g
    for gname, a, b in zip(("dq", "dk", "dv", "dS0"), outs["fused"], outs["separate"]):
        assert torch.equal(a, b), gname


@pytest.mark.parametrize("B,H,N,d,block", [
    (1, 2, 300, 128, 64), (2, 3, 129, 64, 128), (1, 2, 77, 128, 16), (1, 1, 1, 64, 32), (1, 4, 1000, 64, 64),
])
def test_backward_fp32(B, H, N, d, block):
    """fp32 inputs and outputs: the fp32 kernel in the gradient roles, gated
    at 1e-4 like the fp32 forward path."""
    announce("backward fp32", B, H, N, d, block)
    rng = np.random.default_rng([80, N, d])
    q, k, v, dO = (rng.standard_normal((B, H, N, d)).astype(np.float32) * s
                   for s in (d ** -0.5, d ** -0.5, 1.0, 1.0))
    S0 = random_state(N + 2, (B, H), d)
    dSN = random_state(N + 3, (B, H), d)
    ref = oracle.backward(q, k, v, dO, S0, dSN)
    got = gpu_backward(q, k, v, dO, S0, dSN, block, dtype="fp32")
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    print("  rel err dq={:.2e} dk={:.2e} dv={:.2e} dS0={:.2e}".format(*errs))
    assert max(errs) <= 1e-4, errs


def test_backward_fp32_exact_integers_and_edges():
    """Exact integers give the oracle's gradients bitwise; NULL states mean
    zero; with no tokens dS_0 = dS_N."""
    announce("backward fp32 exact integers / edges")
    B, H, N, d = 1, 3, 150, 64
    q, k, v = synth.integer_inputs(990, B, H, N, d)
    dO, _, _ = synth.integer_inputs(991, B, H, N, d)
    rng = np.random.default_rng(92)
    S0 = rng.integers(-2, 3, (B, H, d, d)).astype(np.float64)
    dSN = rng.integers(-2, 3, (B, H, d, d)).astype(np.float64)
    ref = oracle.backward(q, k, v, dO, S0, dSN)
    got = gpu_backward(q, k, v, dO, S0, dSN, 64, dtype="fp32")
    for name, g, r in zip(("dq", "dk", "dv", "dS0"), got, ref):
        np.testing.assert_array_equal(g, r, err_msg=name)
    ref0 = oracle.backward(q, k, v, dO, None, None)
    got0 = gpu_backward(q, k, v, dO, None, None, 64, dtype="fp32")
    for name, g, r in zip(("dq", "dk", "dv", "dS0"), got0, ref0):
        np.testing.assert_array_equal(g, r, err_msg=name)
    e = np.zeros((B, H, 0, d), np.float32)
    _, _, _, dS0 = gpu_backward(e, e, e, e, None, dSN, 64, dtype="fp32")
    np.testing.assert_array_equal(dS0, dSN)
