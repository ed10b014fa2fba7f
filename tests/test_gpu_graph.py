"""The library's launches under HIP graph capture.

Every entry point only validates its arguments and enqueues kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a caller
may capture a sequence of calls in a HIP graph and replay it.  These tests
capture decode steps, a prefill, the sequence-split prefill and the split
state accumulation, replay each graph several times with eager work and
synchronisations between the replays, and require every replay to equal the
eagerly launched result bitwise.
"""
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth

from gpu_helpers import announce

pytestmark = pytest.mark.gpu


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
            t.fill_(float("nan"))
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            assert torch.equal(t, r), f"replay {i} differs from the eager run"
        reset()
        run()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            assert torch.equal(t, r), f"eager run after replay {i} differs"


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
