"""GPU parity of the draft-verification step (outputs of T draft tokens from
one read of the state, state untouched) and of the commit of the accepted
drafts, against the fp64 oracle and against one-token decode steps."""
import numpy as np
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth
from oracle import oracle

from gpu_helpers import announce, dev, host, random_state, rel_err

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}


def bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def drafts(seed, B, H, T, d, dtype):
    q, k, v = synth.prefill_inputs(seed, B, H, T, d, dtype)
    return q, k, v


@pytest.mark.parametrize("B,H,T,d,io", [
    (2, 3, 1, 128, "bf16"), (2, 3, 4, 128, "bf16"), (1, 5, 16, 128, "bf16"), (3, 2, 7, 64, "bf16"),
    (2, 2, 16, 64, "fp32"), (1, 3, 5, 128, "fp32"),
    # draft counts below the room of their variant (4, 8, 16), both I/O types
    (2, 3, 13, 128, "fp32"), (2, 5, 9, 128, "bf16"), (1, 3, 12, 64, "bf16"), (3, 3, 6, 128, "fp32"),
    # room for 4 drafts at d = 64 (one pipelined batch per wave)
    (2, 3, 3, 64, "bf16"), (1, 5, 4, 64, "fp32"),
])
def test_verify_matches_oracle_and_leaves_state(B, H, T, d, io):
    announce("decode verify", B, H, T, d, io)
    q, k, v = drafts(40 + T, B, H, T, d, io)
    S0 = random_state(T + d, (B, H), d, scale=3.0)
    o_ref, _ = oracle.recurrence(q, k, v, S0)
    Sd = torch.from_numpy(S0).cuda()
    before = Sd.clone()
    od = torch.empty((B, H, T, d), dtype=dev(q, io).dtype, device="cuda")
    la.decode_verify(dev(q, io), dev(k, io), dev(v, io), od, Sd)
    torch.cuda.synchronize()
    assert torch.equal(Sd, before)
    e = rel_err(host(od), o_ref)
    print(f"  rel err o={e:.3e}")
    assert e <= TOL[io]


@pytest.mark.parametrize("d", [64, 128])
def test_verify_bf16_state(d):
    """With a bf16 state the outputs follow the oracle run from the stored
    (bf16) state, which the kernel widens exactly."""
    announce("decode verify bf16 state", d)
    B, H, T = 2, 3, 8
    q, k, v = drafts(50, B, H, T, d, "bf16")
    S0 = random_state(d, (B, H), d, scale=3.0)
    Sb = torch.from_numpy(S0).to(torch.bfloat16).cuda()
    S_stored = oracle.bf16_bits_to_f64(bf16_bits(Sb))
    o_ref, _ = oracle.recurrence(q, k, v, S_stored)
    od = torch.empty((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    la.decode_verify(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), od, Sb)
    torch.cuda.synchronize()
    assert rel_err(host(od), o_ref) <= TOL["bf16"]


@pytest.mark.parametrize("d,io", [(128, "bf16"), (64, "bf16"), (128, "fp32")])
def test_commit_equals_decode_steps(d, io):
    """An fp32-state commit of a_b drafts is bit-identical to a_b one-token
    decode steps, and matches the oracle's state after the accepted prefix.
    Out-of-range counts are clamped to [0, T]."""
    announce("decode commit", d, io)
    B, H, T = 6, 2, 9
    q, k, v = drafts(60, B, H, T, d, io)
    S0 = random_state(11, (B, H), d, scale=2.0)
    accept = np.array([0, 1, 4, T, -3, T + 7], dtype=np.int32)
    eff = np.clip(accept, 0, T)
    Sd = torch.from_numpy(S0).cuda()
    la.decode_commit(dev(k, io), dev(v, io), Sd, torch.from_numpy(accept).cuda())
    # reference 1: one-token decode steps, batch entry by batch entry
    for b in range(B):
        Sb = torch.from_numpy(np.ascontiguousarray(S0[b:b + 1])).cuda()
        od = torch.empty((1, H, d), dtype=dev(q[:1, :, 0], io).dtype, device="cuda")
        for t in range(int(eff[b])):
            la.decode(dev(q[b:b + 1, :, t], io), dev(k[b:b + 1, :, t], io), dev(v[b:b + 1, :, t], io), od, Sb)
        torch.cuda.synchronize()
        assert torch.equal(Sd[b:b + 1], Sb), b
    # reference 2: the oracle's state after the accepted prefix
    for b in range(B):
        a = int(eff[b])
        _, S_ref = oracle.recurrence(q[b:b + 1, :, :a], k[b:b + 1, :, :a], v[b:b + 1, :, :a], S0[b:b + 1])
        assert rel_err(host(Sd[b:b + 1]), S_ref) <= 1e-5, b


def test_commit_all_and_bf16_state():
    """accept = NULL commits every draft; a bf16 state is updated in fp32 and
    rounded once, within one bf16 step of the oracle's rounding of the exact
    update."""
    announce("decode commit all / bf16 state")
    B, H, T, d = 2, 3, 12, 128
    q, k, v = drafts(70, B, H, T, d, "bf16")
    S0 = synth.decode_initial_state(B, H, d, n_outer=256)
    Sb = torch.from_numpy(S0).to(torch.bfloat16).cuda()
    S_stored = oracle.bf16_bits_to_f64(bf16_bits(Sb))
    la.decode_commit(dev(k, "bf16"), dev(v, "bf16"), Sb)
    torch.cuda.synchronize()
    _, S_exact = oracle.recurrence(q, k, v, S_stored)
    want = oracle.bf16_bits_to_f64(oracle.round_bf16_bits(S_exact))
    got = oracle.bf16_bits_to_f64(bf16_bits(Sb))
    ulp = np.maximum(np.abs(want), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(got - want) <= ulp)
    assert np.mean(got == want) > 0.99


def test_verify_then_commit_matches_decode_outputs():
    """Draft outputs from verify agree with T one-token decode steps."""
    announce("verify vs decode steps")
    B, H, T, d = 2, 4, 6, 128
    q, k, v = drafts(80, B, H, T, d, "bf16")
    S0 = random_state(13, (B, H), d, scale=2.0)
    Sd = torch.from_numpy(S0).cuda()
    ov = torch.empty((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    la.decode_verify(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), ov, Sd)
    S2 = torch.from_numpy(S0).cuda()
    od = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    outs = []
    for t in range(T):
        la.decode(dev(q[:, :, t], "bf16"), dev(k[:, :, t], "bf16"), dev(v[:, :, t], "bf16"), od, S2)
        outs.append(host(od))
    torch.cuda.synchronize()
    assert rel_err(host(ov), np.stack(outs, axis=2)) <= 1e-2
    la.decode_commit(dev(k, "bf16"), dev(v, "bf16"), Sd)
    torch.cuda.synchronize()
    assert torch.equal(Sd, S2)


@pytest.mark.parametrize("d", [128, 64])
def test_commit_odd_head_count_equals_decode_steps(d):
    """Seven sequences with an fp32 state: the commit's last workgroup holds
    one head and a pair of idle waves; its state is still bit-identical to
    the accepted drafts' decode steps."""
    announce("decode commit odd head count", d)
    B, H, T = 7, 1, 5
    q, k, v = drafts(61, B, H, T, d, "bf16")
    S0 = random_state(12, (B, H), d, scale=2.0)
    accept = np.array([5, 0, 3, 1, 4, 2, 5], dtype=np.int32)
    Sd = torch.from_numpy(S0).cuda()
    la.decode_commit(dev(k, "bf16"), dev(v, "bf16"), Sd, torch.from_numpy(accept).cuda())
    Sb = torch.from_numpy(S0).cuda()
    for b in range(B):
        od = torch.empty((1, H, d), dtype=torch.bfloat16, device="cuda")
        Sv = Sb[b:b + 1]
        for t in range(int(accept[b])):
            la.decode(dev(q[b:b + 1, :, t], "bf16"), dev(k[b:b + 1, :, t], "bf16"), dev(v[b:b + 1, :, t], "bf16"),
                      od, Sv)
    torch.cuda.synchronize()
    assert torch.equal(Sd, Sb)
