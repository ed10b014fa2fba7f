"""The library's launches under HIP graph capture.

Every entry point only validates its arguments and enqueues kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a caller
may capture a sequence of calls in a HIP graph and replay it.  These tests
capture decode steps, a prefill, the sequence-split prefill, the split
state accumulation, the fused backward, speculative verify and commit and
a scaled E4M3 decode, replay each graph several times with eager work and
synchronisations between the replays, and require every replay to equal the
eagerly launched result bitwise.
"""
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth

from gpu_helpers import announce

pytestmark = pytest.mark.gpu


def same(a, b):
    if a.dtype == torch.float8_e4m3fn:
        return torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    return torch.equal(a, b)


def replay_check(run, outputs, reset):
    """Eager reference, one capture, then three replays each followed by an
    eager run; every replay's outputs must equal the reference bitwise."""
    reset()
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        # poison every output, then restore the inputs the run reads (states)
        for t in outputs:
            if t.dtype == torch.float8_e4m3fn:
                t.view(torch.uint8).fill_(0x7f)  # E4M3 NaN
            else:
                t.fill_(float("nan"))
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            assert same(t, r), f"replay {i} differs from the eager run"
        reset()
        run()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            assert same(t, r), f"eager run after replay {i} differs"


def test_graph_decode_steps():
    announce("graph: 8 decode steps, 16 x 8 sequences, fp32 and bf16 state")
    B, H, d, T = 16, 8, 128, 8
    S0 = synth.decode_initial_state_device(B, H, d, n_outer=64)
    inputs = [synth.decode_step_inputs_device(t, B, H, d) for t in range(T)]
    o = torch.empty((T, B, H, d), dtype=torch.bfloat16, device="cuda")
    for S_init in (S0, S0.to(torch.bfloat16)):
        S = S_init.clone()

        def run():
            for t, (q, k, v) in enumerate(inputs):
                la.decode(q, k, v, o[t], S)

        replay_check(run, [S, o], lambda: S.copy_(S_init))


def test_graph_prefill_and_seqsplit():
    announce("graph: prefill, sequence-split prefill, split state accumulation")
    B, H, N, d = 1, 4, 4096, 128
    q, k, v = synth.prefill_inputs_device(31, B, H, N, d)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator(device="cuda").manual_seed(31), device="cuda")
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    S1, S2, dS = S0.clone(), S0.clone(), torch.zeros_like(S0)
    ws_p = torch.empty(max(16, la.prefill_seqsplit_workspace(B, H, N, d, 128, torch.bfloat16)),
                       dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(max(16, la.state_accumulate_split_workspace(B, H, N, d, torch.bfloat16)),
                       dtype=torch.uint8, device="cuda")
    assert ws_p.numel() > 16 and ws_s.numel() > 16

    def reset():
        S1.copy_(S0)
        S2.copy_(S0)
        dS.zero_()

    def run():
        la.prefill(q, k, v, o1, S1, 128)
        la.prefill_seqsplit(q, k, v, o2, S2, 128, ws_p)
        la.state_accumulate_split(k, v, dS, ws_s)

    replay_check(run, [o1, S1, o2, S2, dS], reset)


def test_graph_backward_and_speculative():
    announce("graph: fused backward, speculative verify/commit, scaled E4M3 decode")
    B, H, N, d = 1, 4, 1000, 128
    q, k, v = synth.prefill_inputs_device(32, B, H, N, d)
    dO = synth.prefill_inputs_device(33, B, H, N, d)[2]
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ds0 = torch.empty((B, H, d, d), device="cuda")
    dSN = torch.randn((B, H, d, d), generator=torch.Generator(device="cuda").manual_seed(33), device="cuda")

    def run_bwd():
        la.backward(q, k, v, dO, dq, dk, dv, 128, dstate=dSN, dstate0=ds0, strategy=la.BWD_FUSED)

    replay_check(run_bwd, [dq, dk, dv, ds0], lambda: None)

    Bd, Hd, T = 8, 4, 4
    S0 = synth.decode_initial_state_device(Bd, Hd, d, n_outer=64)
    tq, tk, tv = synth.prefill_inputs_device(34, Bd, Hd, T, d)
    to = torch.empty_like(tq)
    acc = torch.tensor([3, 0, 4, 1, 2, 4, 3, 1], dtype=torch.int32, device="cuda")
    S = S0.clone()
    scale = torch.exp2(torch.ceil(torch.log2(S0.abs().amax(dim=(2, 3)) / 224.0)))
    S8_0 = (S0 / scale[:, :, None, None]).to(torch.float8_e4m3fn)
    S8 = S8_0.clone()
    dq1, dk1, dv1 = synth.decode_step_inputs_device(3, Bd, Hd, d)
    o1 = torch.empty_like(dq1)

    def run_spec():
        la.decode_verify(tq, tk, tv, to, S)
        la.decode_commit(tk, tv, S, acc)
        la.decode(dq1, dk1, dv1, o1, S8, state_scale=scale)

    def reset():
        S.copy_(S0)
        S8.copy_(S8_0)

    replay_check(run_spec, [to, S, o1, S8], reset)
