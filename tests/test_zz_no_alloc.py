"""GPU checks of ``lin_attn_prefill_seqsplit_noalloc``: the sequence-split
prefill with its workspace in the library's fixed per-device scratch buffer.

The entry point runs the same plan and kernels as ``lin_attn_prefill_seqsplit``
with a caller workspace, so its outputs and final states must be bitwise
equal to that call's on the same inputs.  Calls follow one another on one
stream, largest first, so a later, smaller call runs over the leftovers of
an earlier one in the shared buffer; the smallest case is also checked
against the fp64 oracle (max|gpu - oracle| / max|oracle| <= 1e-2 for bf16
inputs with an fp32 state).  A plan that needs more workspace than the
buffer holds is refused before any launch.
"""
import numpy as np
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth
from oracle import oracle

from gpu_helpers import announce, host, random_state, rel_err

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2


def run_both(B, H, N, d, block, seed):
    """(o, S) of the workspace entry point and of the scratch entry point on
    the same device-generated inputs and a random S_0."""
    q, k, v = synth.prefill_inputs_device(seed, B, H, N, d)
    S0 = torch.from_numpy(random_state(seed, (B, H), d)).cuda()
    need = la.prefill_seqsplit_workspace(B, H, N, d, block, torch.bfloat16)
    announce("seqsplit noalloc", B, H, N, d, block, f"workspace {need} of scratch {la.scratch_bytes()}")
    assert 0 < need <= la.scratch_bytes(), "the case must cut the sequences and fit the scratch buffer"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws, S_ws = torch.empty_like(q), S0.clone()
    la.prefill_seqsplit(q, k, v, o_ws, S_ws, block, ws)
    o_sc, S_sc = torch.full_like(q, float("nan")), S0.clone()
    la.prefill_seqsplit_noalloc(q, k, v, o_sc, S_sc, block)
    torch.cuda.synchronize()
    return (q, k, v, S0), (o_ws, S_ws), (o_sc, S_sc)


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    # largest plan first, then smaller ones over its leftovers in the buffer:
    #  - one sequence of 2^19 tokens: 256 parts of 2048, two launches (state
    #    pass in 2 chunks per part): 511 states, 31.9 MiB;
    #  - the 1M-token sequence's shard (64 sequences x 131072 tokens, 4 parts,
    #    one launch): 24 MiB;
    #  - 8 sequences x 8192 tokens (32 parts, one launch) and 2 x 4096 at d = 64
    cases = [(1, 1, 1 << 19, 128, 128, 60), (1, 64, 131072, 128, 128, 61), (1, 8, 8192, 128, 128, 62),
             (1, 2, 4096, 64, 64, 63)]
    for i, (B, H, N, d, block, seed) in enumerate(cases):
        inputs, (o_ws, S_ws), (o_sc, S_sc) = run_both(B, H, N, d, block, seed)
        assert torch.equal(o_sc, o_ws), f"call {i}: outputs differ from the workspace entry point"
        assert torch.equal(S_sc, S_ws), f"call {i}: final states differ from the workspace entry point"
        if i == len(cases) - 1:
            q, k, v, S0 = (host(t) for t in inputs)
            o_ref, S_ref = oracle.recurrence(q, k, v, S0)
            eo, es = rel_err(host(o_sc), o_ref), rel_err(host(S_sc), S_ref)
            print(f"  call {i} vs oracle: o {eo:.3e}, state {es:.3e}")
            assert eo <= TOL_BF16 and es <= TOL_BF16


def test_noalloc_uncut_case_needs_no_scratch():
    """Enough sequences to fill the GPU: no cut, the plain prefill runs."""
    B, H, N, d, block = 2, 256, 512, 64, 64
    announce("seqsplit noalloc uncut", B, H, N, d, block)
    assert la.prefill_seqsplit_workspace(B, H, N, d, block, torch.bfloat16) == 0
    q, k, v = synth.prefill_inputs_device(64, B, H, N, d)
    S0 = torch.from_numpy(random_state(64, (B, H), d)).cuda()
    o1, S1 = torch.empty_like(q), S0.clone()
    la.prefill(q, k, v, o1, S1, block)
    o2, S2 = torch.empty_like(q), S0.clone()
    la.prefill_seqsplit_noalloc(q, k, v, o2, S2, block)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_noalloc_refuses_a_plan_larger_than_the_scratch():
    """One sequence of 2^21 tokens at d = 128 is cut into as many parts as
    the GPU has compute units, each summed in 4 chunks: on a 256-unit device
    that plan needs 63.8 MiB, more than the 56 MiB buffer; the call returns
    LIN_ATTN_ESCRATCH before any launch and leaves its outputs untouched."""
    B, H, N, d, block = 1, 1, 1 << 21, 128, 128
    need = la.prefill_seqsplit_workspace(B, H, N, d, block, torch.bfloat16)
    announce("seqsplit noalloc refusal", B, H, N, d, block, f"workspace {need}")
    if need <= la.scratch_bytes():
        pytest.skip(f"this device's plan needs only {need} bytes")
    q, k, v = (torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o = torch.full_like(q, 3.0)
    S = torch.full((B, H, d, d), 5.0, device="cuda")
    with pytest.raises(la.LinAttnError) as e:
        la.prefill_seqsplit_noalloc(q, k, v, o, S, block)
    assert e.value.code == la.ESCRATCH
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((S == 5.0).all())
