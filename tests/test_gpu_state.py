"""GPU parity of the state accumulation over a token segment
(``lin_attn_state_accumulate``: state += K^T V) against the fp64 oracle, and
of the sequence-parallel recombination it serves: segments processed
independently, their K^T V prefix-summed into each segment's initial state,
reproduce the prefill of the whole sequence.

Gates as for the prefill: max|gpu - oracle| / max|oracle| <= 1e-2 (bf16
inputs, fp32 state) and <= 1e-4 (fp32 inputs); exact for exact-integer inputs.
"""
import numpy as np
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth
from oracle import oracle

from gpu_helpers import announce, dev, gpu_prefill, host, random_state, rel_err

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_F32 = 1e-4


def gpu_accumulate(k, v, S0, dtype):
    kd, vd = dev(k, dtype), dev(v, dtype)
    Sd = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    la.state_accumulate(kd, vd, Sd)
    torch.cuda.synchronize()
    return host(Sd)


def oracle_state(k, v, S0):
    q = np.zeros_like(k)
    return oracle.recurrence(q, k, v, S0)[1]


@pytest.mark.parametrize("d,N", [(128, 1), (128, 77), (128, 128), (128, 300), (64, 129), (64, 1000)])
def test_state_accumulate_exact_integers(d, N):
    announce("state accumulate exact-integer", d, N)
    _, k, v = synth.integer_inputs(3000 + d + N, 1, 2, N, d)
    rng = np.random.default_rng([5, d, N])
    S0 = rng.integers(-2, 3, size=(1, 2, d, d)).astype(np.float32)
    abs_s = np.abs(S0).astype(np.float64) + np.einsum("bhti,bhtj->bhij", np.abs(k), np.abs(v))
    assert abs_s.max() <= 256, "integer case leaves the exact range"
    np.testing.assert_array_equal(gpu_accumulate(k, v, S0, "bf16"), oracle_state(k, v, S0))
    np.testing.assert_array_equal(gpu_accumulate(k, v, S0, "fp32"), oracle_state(k, v, S0))


@pytest.mark.parametrize("B,H,N,d,dtype", [
    (1, 3, 1000, 128, "bf16"), (2, 8, 257, 128, "bf16"), (1, 2, 5, 64, "bf16"), (2, 2, 700, 64, "bf16"),
    (1, 2, 300, 128, "fp32"), (1, 3, 130, 64, "fp32"),
])
def test_state_accumulate_random(B, H, N, d, dtype):
    announce("state accumulate random", B, H, N, d, dtype)
    _, k, v = synth.prefill_inputs(20, B, H, N, d, dtype)
    S0 = random_state(N + d, (B, H), d, scale=2.0)
    S = gpu_accumulate(k, v, S0, dtype)
    err = rel_err(S, oracle_state(k, v, S0))
    print(f"  rel err state={err:.3e}")
    assert err <= (TOL_BF16 if dtype == "bf16" else TOL_F32)


def test_state_accumulate_deterministic_and_empty():
    announce("state accumulate determinism / N=0")
    _, k, v = synth.prefill_inputs(21, 1, 8, 900, 128, "bf16")
    S0 = random_state(1, (1, 8), 128)
    runs = [gpu_accumulate(k, v, S0, "bf16") for _ in range(3)]
    for r in runs[1:]:
        np.testing.assert_array_equal(r, runs[0])
    kd = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    Sd = torch.randn((1, 2, 128, 128), device="cuda")
    before = Sd.clone()
    la.state_accumulate(kd, kd, Sd)
    torch.cuda.synchronize()
    assert torch.equal(Sd, before)


@pytest.mark.parametrize("G,d,block", [(4, 128, 128), (3, 64, 64)])
def test_sequence_parallel_recombination(G, d, block):
    """Cut a sequence into G segments (ragged lengths); accumulate each
    segment's K^T V from zero, prefix-sum them (exclusive) onto S_0, and run
    each segment's prefill from its sum: outputs and final state match the
    oracle of the whole sequence."""
    announce("sequence-parallel recombination", G, d, block)
    B, H, N = 1, 2, 1000
    q, k, v = synth.prefill_inputs(22, B, H, N, d, "bf16")
    S0 = random_state(9, (B, H), d)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    cuts = {4: [0, 137, 500, 733, N], 3: [0, 300, 701, N]}[G]
    deltas = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        deltas.append(gpu_accumulate(k[:, :, a:b], v[:, :, a:b], np.zeros((B, H, d, d), np.float32), "bf16"))
    start = S0.astype(np.float64)
    outs = []
    S_last = None
    for (a, b), dS in zip(zip(cuts[:-1], cuts[1:]), deltas):
        o_seg, S_seg = gpu_prefill(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], start.astype(np.float32), block, "bf16")
        outs.append(o_seg)
        start = start + dS
        S_last = S_seg
    o_cat = np.concatenate(outs, axis=2)
    eo, es, ed = rel_err(o_cat, o_ref), rel_err(S_last, S_ref), rel_err(start, S_ref)
    print(f"  rel err o={eo:.3e} state(prefill)={es:.3e} state(sum of deltas)={ed:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16 and ed <= TOL_BF16


# ---- token-split accumulation (lin_attn_state_accumulate_split) ----

def gpu_accumulate_split(k, v, S0, dtype, workspace=None):
    kd, vd = dev(k, dtype), dev(v, dtype)
    Sd = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    la.state_accumulate_split(kd, vd, Sd, workspace)
    torch.cuda.synchronize()
    return host(Sd)


@pytest.mark.parametrize("H,N,d", [(2, 1000, 128), (1, 2000, 64), (1, 257, 128), (3, 4099, 128), (2, 64, 64)])
def test_state_accumulate_split_exact_integers(H, N, d):
    """Sparse {-1, 0, 1} inputs: every partial and chunk sum is an exact
    integer in fp32, so the split accumulation equals the oracle bitwise,
    whatever the chunking (several chunks, a ragged last chunk and stage,
    and a single chunk)."""
    announce("state accumulate split exact-integer", H, N, d)
    _, k, v = synth.integer_inputs(3100 + d + N, 1, H, N, d)
    rng = np.random.default_rng([6, d, N])
    S0 = rng.integers(-2, 3, size=(1, H, d, d)).astype(np.float32)
    ref = oracle_state(k, v, S0)
    assert np.abs(ref).max() < 2 ** 24
    np.testing.assert_array_equal(gpu_accumulate_split(k, v, S0, "bf16"), ref)


@pytest.mark.parametrize("B,H,N,d", [(1, 3, 5000, 128), (2, 4, 3000, 64), (1, 1, 20000, 128), (4, 64, 300, 128)])
def test_state_accumulate_split_random(B, H, N, d):
    announce("state accumulate split random", B, H, N, d)
    _, k, v = synth.prefill_inputs(23, B, H, N, d, "bf16")
    S0 = random_state(N + 7, (B, H), d, scale=2.0)
    chunks_ws = la.state_accumulate_split_workspace(B, H, N, d, torch.bfloat16)
    S = gpu_accumulate_split(k, v, S0, "bf16")
    err = rel_err(S, oracle_state(k, v, S0))
    # the same sum through the tile kernel, up to fp32 rounding
    S_tile = gpu_accumulate(k, v, S0, "bf16")
    err_tile = rel_err(S, S_tile)
    print(f"  workspace {chunks_ws} B; rel err state={err:.3e}; vs tile kernel {err_tile:.3e}")
    assert err <= TOL_BF16
    assert err_tile <= 1e-5


def test_state_accumulate_split_deterministic_workspace_and_fp32():
    """Bitwise repeatable (the chunk sums are added in a fixed order);
    a workspace one element short is rejected before any launch, a larger
    one is accepted; N = 0 changes nothing; fp32 inputs take the unsplit
    kernel and need no workspace."""
    announce("state accumulate split determinism / workspace / fp32")
    B, H, N, d = 1, 4, 6000, 128
    _, k, v = synth.prefill_inputs(24, B, H, N, d, "bf16")
    S0 = random_state(2, (B, H), d)
    need = la.state_accumulate_split_workspace(B, H, N, d, torch.bfloat16)
    assert need > 0
    runs = [gpu_accumulate_split(k, v, S0, "bf16") for _ in range(3)]
    for r in runs[1:]:
        np.testing.assert_array_equal(r, runs[0])
    big = torch.full((need + 4096,), 7, dtype=torch.uint8, device="cuda")
    np.testing.assert_array_equal(gpu_accumulate_split(k, v, S0, "bf16", big), runs[0])
    short = torch.empty((need - 1,), dtype=torch.uint8, device="cuda")
    kd, vd = dev(k, "bf16"), dev(v, "bf16")
    Sd = torch.from_numpy(S0.astype(np.float32)).cuda()
    with pytest.raises(la.LinAttnError):
        la.state_accumulate_split(kd, vd, Sd, short)
    e = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    Se = torch.randn((1, 2, 128, 128), device="cuda")
    before = Se.clone()
    la.state_accumulate_split(e, e, Se)
    torch.cuda.synchronize()
    assert torch.equal(Se, before)
    assert la.state_accumulate_split_workspace(1, 2, 3000, 64, torch.float32) == 0
    _, k32, v32 = synth.prefill_inputs(25, 1, 2, 3000, 64, "fp32")
    S32 = random_state(3, (1, 2), 64)
    assert rel_err(gpu_accumulate_split(k32, v32, S32, "fp32"), oracle_state(k32, v32, S32)) <= TOL_F32


def test_state_accumulate_split_shard_workload_sampled():
    """One segment of the 1M-token sequence cut 8 ways (B=1, H=64,
    N=131072, d=128): all 64 heads on the GPU in the launch configuration
    the benchmark times, two heads checked against the oracle."""
    announce("state accumulate split shard workload B=1 H=64 N=131072 sampled")
    B, H, N, d = 1, 64, 131072, 128
    _, k, v = synth.prefill_inputs_device(4, B, H, N, d)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    la.state_accumulate_split(k, v, S)
    S_tile = torch.zeros_like(S)
    la.state_accumulate(k, v, S_tile)
    torch.cuda.synchronize()
    assert rel_err(host(S), host(S_tile)) <= 1e-5
    for h in (3, 61):
        kh, vh = host(k[:, h:h + 1]), host(v[:, h:h + 1])
        err = rel_err(host(S[:, h:h + 1]), oracle.state_after(kh, vh))
        print(f"  head {h} rel err state={err:.3e}")
        assert err <= TOL_BF16
