"""GPU parity of the prefill cut along the tokens (``lin_attn_prefill_seqsplit``)
against the fp64 oracle.

Each sequence's tokens are cut into P parts; the parts' initial states come
from the K^T V of the parts before them (the token-split accumulation plus an
ordered prefix sum), and the parts run as independent chunked prefills.  The
outputs and the final state are those of the whole sequence.

Gates as for the prefill: max|gpu - oracle| / max|oracle| <= 1e-2 (bf16
inputs, fp32 state); exact for exact-integer inputs.
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


def gpu_seqsplit(q, k, v, S0, block, dtype="bf16", workspace=None):
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    od = torch.full_like(qd, float("nan"))
    Sd = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    la.prefill_seqsplit(qd, kd, vd, od, Sd, block, workspace)
    torch.cuda.synchronize()
    return host(od), host(Sd)


@pytest.mark.parametrize("B,H,N,d,block", [
    (1, 4, 16384, 128, 128),   # 32 parts of 512
    (2, 2, 8192, 64, 64),      # 16 parts
    (1, 1, 4176, 128, 128),    # 8 parts of 522: ragged last block in every part
    (1, 3, 12288, 128, 64),    # 16 parts of 768
    (1, 1, 65536, 128, 128),   # 64 parts of 1024, 1 accumulation chunk each
    (1, 2, 16384, 64, 128),    # 32 parts of 512 (d = 64)
])
def test_seqsplit_random(B, H, N, d, block):
    ws = la.prefill_seqsplit_workspace(B, H, N, d, block, torch.bfloat16)
    announce("prefill seqsplit random", B, H, N, d, block, f"workspace {ws}")
    assert ws > 0, "the case must cut the sequences"
    q, k, v = synth.prefill_inputs(40 + N % 97, B, H, N, d)
    S0 = random_state(N, (B, H), d)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    o, S = gpu_seqsplit(q, k, v, S0, block)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    o1, S1 = gpu_prefill(q, k, v, S0, block, "bf16")
    print(f"  rel err o={eo:.3e} state={es:.3e}; uncut prefill o={rel_err(o1, o_ref):.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("H,N,d,block", [(2, 4096, 128, 128), (1, 8192, 64, 64), (3, 6144, 128, 96)])
def test_seqsplit_exact_integers(H, N, d, block):
    """Sparse {-1, 0, 1} inputs keep every state entry, partial sum and
    output an exact integer within bf16's range: the cut prefill equals the
    oracle bitwise (part boundaries, the ordered prefix of part states and
    the last part's final state are all exercised)."""
    assert la.prefill_seqsplit_workspace(1, H, N, d, block, torch.bfloat16) > 0
    announce("prefill seqsplit exact integers", H, N, d, block)
    q, k, v = synth.integer_inputs(4100 + N + d, 1, H, N, d)
    rng = np.random.default_rng([41, N, d])
    S0 = rng.integers(-2, 3, size=(1, H, d, d)).astype(np.float32)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    assert np.abs(o_ref).max() <= 256 and np.abs(S_ref).max() <= 256, "integer case leaves bf16's exact range"
    o, S = gpu_seqsplit(q, k, v, S0, block)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(S, S_ref)


def test_seqsplit_uncut_cases_and_workspace():
    """When no cut is made (enough sequences, or too few tokens) the call is
    the plain prefill, bitwise; a workspace one byte short is rejected; a
    cut call is bitwise repeatable."""
    announce("prefill seqsplit uncut / workspace / determinism")
    q, k, v = synth.prefill_inputs(42, 2, 2, 1000, 128)  # 1000 tokens: no cut (parts of 500 < 512)
    S0 = random_state(3, (2, 2), 128)
    assert la.prefill_seqsplit_workspace(2, 2, 1000, 128, 128, torch.bfloat16) == 0
    o, S = gpu_seqsplit(q, k, v, S0, 128)
    o1, S1 = gpu_prefill(q, k, v, S0, 128, "bf16")
    np.testing.assert_array_equal(o, o1)  # no cut: the plain prefill, bitwise
    np.testing.assert_array_equal(S, S1)
    assert la.prefill_seqsplit_workspace(4, 64, 32768, 128, 128, torch.bfloat16) == 0  # 256 sequences
    assert la.prefill_seqsplit_workspace(1, 2, 8192, 128, 64, torch.float32) == 0
    B, H, N, d = 1, 2, 8192, 128
    q, k, v = synth.prefill_inputs(43, B, H, N, d)
    need = la.prefill_seqsplit_workspace(B, H, N, d, 128, torch.bfloat16)
    assert need > 0
    runs = [gpu_seqsplit(q, k, v, S0[:1], 128) for _ in range(2)]
    for a, b in zip(*runs):
        np.testing.assert_array_equal(a, b)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    od = torch.empty_like(qd)
    Sd = torch.zeros((B, H, d, d), device="cuda")
    with pytest.raises(la.LinAttnError):
        la.prefill_seqsplit(qd, kd, vd, od, Sd, 128, torch.empty(need - 1, dtype=torch.uint8, device="cuda"))


def test_seqsplit_shard_workload_sampled():
    """One of 8 segments of the 1M-token sequence (B=1, H=64, N=131072,
    d=128, block 128) from a non-zero S_0, as the benchmark runs it: every
    head against the uncut prefill on the GPU, two heads against the oracle."""
    announce("prefill seqsplit shard workload B1 H64 N131072 (heads 0, 45 vs oracle)")
    B, H, N, d = 1, 64, 131072, 128
    heads = [(0, 0), (0, 45)]
    q, k, v = synth.prefill_inputs_device(6, B, H, N, d)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator(device="cuda").manual_seed(6),
                     device="cuda", dtype=torch.float32)
    S = S0.clone()
    o = torch.empty_like(q)
    la.prefill_seqsplit(q, k, v, o, S, 128)
    S_u = S0.clone()
    o_u = torch.empty_like(q)
    la.prefill(q, k, v, o_u, S_u, 128)
    torch.cuda.synchronize()
    d_o = (o.float() - o_u.float()).abs().max().item() / o_u.float().abs().max().item()
    d_s = (S - S_u).abs().max().item() / S_u.abs().max().item()
    print(f"  cut vs uncut prefill, all heads: o {d_o:.3e} state {d_s:.3e}", flush=True)
    assert d_o <= TOL_BF16 and d_s <= 1e-4
    qh, kh, vh = (np.stack([t[b, h].float().cpu().numpy() for b, h in heads]) for t in (q, k, v))
    S0h = np.stack([host(S0[b, h]) for b, h in heads])
    oh = np.stack([host(o[b, h]) for b, h in heads])
    Sh = np.stack([host(S[b, h]) for b, h in heads])
    del q, k, v, o, o_u
    torch.cuda.empty_cache()
    o_ref, S_ref = oracle.recurrence(qh, kh, vh, S0h)
    eo, es = rel_err(oh, o_ref), rel_err(Sh, S_ref)
    print(f"  heads {heads}: rel err o={eo:.3e} state={es:.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16
