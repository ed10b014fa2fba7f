"""GPU parity of the prefill cut along the tokens (``lin_attn_prefill_seqsplit``)
against the fp64 oracle.

Each sequence's tokens are cut into P parts; the parts' initial states come
from the K^T V of the parts before them, added in part order, and the parts
run as independent chunked prefills.  At d = 128, up to 32 parts per
sequence form those starts in the same launch (each part publishes its own
K^T V behind a flag, then the parts form the starts together); otherwise a
separate token-split state pass runs first.  The outputs and the final state are those of
the whole sequence.

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
    (1, 4, 16384, 128, 128),   # 64 parts of 256: two launches
    (2, 2, 8192, 64, 64),      # 32 parts of 256: two launches (d = 64)
    (1, 1, 4176, 128, 128),    # 16 parts of 261: one launch, ragged last block in every part
    (1, 3, 12288, 128, 64),    # 32 parts of 384: one launch, 3 sequences
    (1, 1, 65536, 128, 128),   # 256 parts of 256: two launches, 1 state-pass chunk each
    (1, 2, 16384, 64, 128),    # 64 parts of 256 (d = 64): two launches
    (1, 32, 32768, 64, 64),    # 8 parts of 4096: two launches, 4 state-pass chunks per part
    (1, 32, 32768, 128, 128),  # 8 parts of 4096: one launch, 32 blocks per part
    (1, 4, 20480, 128, 128),   # 64 parts of 320: two launches, ragged last block in every part
    (2, 64, 1024, 128, 128),   # 2 parts of 512: one launch, the smallest cut
    (1, 8, 4096, 128, 32),     # 16 parts of 256, block 32: one launch, 8 blocks held in the staging ring
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
    q, k, v = synth.prefill_inputs(42, 2, 2, 500, 128)  # 500 tokens: no cut (parts of 250 < 256)
    S0 = random_state(3, (2, 2), 128)
    assert la.prefill_seqsplit_workspace(2, 2, 500, 128, 128, torch.bfloat16) == 0
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


def test_seqsplit_one_launch_workspace_contents_do_not_matter():
    """A one-launch cut (B=1 H=8 N=4096 d=128 block 64: 16 parts of 256
    tokens) gives the same result, bitwise, from a zeroed workspace, from one
    full of random bytes and from the workspace a previous call left; each
    call leaves the flag words it used zero (those of parts 0 .. P-2 in the
    value slices its parts run in; the last part has no flag)."""
    B, H, N, d, blk = 1, 8, 4096, 128, 64
    P = 16
    sums = (P - 1) * B * H * d * d * 4
    need = la.prefill_seqsplit_workspace(B, H, N, d, blk, torch.bfloat16)
    announce("prefill seqsplit one launch, workspace contents", B, H, N, d, blk, f"workspace {need}")
    assert need == 2 * sums + B * H * P * 3 * 4 * 8
    q, k, v = synth.prefill_inputs_device(44, B, H, N, d)
    S0 = torch.from_numpy(random_state(44, (B, H), d)).cuda()
    g = torch.Generator(device="cuda").manual_seed(44)
    workspaces = [torch.zeros(need, dtype=torch.uint8, device="cuda"),
                  torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nsplit = 1
    while nsplit < 4 and B * H * P * nsplit < cus:
        nsplit *= 2
    results = []
    for ws in workspaces + [workspaces[1]]:
        o, S = torch.empty_like(q), S0.clone()
        la.prefill_seqsplit(q, k, v, o, S, blk, ws)
        torch.cuda.synchronize()
        flags = ws[2 * sums:].view(torch.int64).view(3, B * H, P, 4)  # published, slab, done
        used = torch.cat([flags[0, :, :P - 1, :nsplit].flatten(), flags[1, :, :, :nsplit].flatten(),
                          flags[2, :, :P - 1, :nsplit].flatten()])
        assert not torch.any(used), f"flag words left set: {torch.nonzero(flags).tolist()[:8]}"
        results.append((o, S))
    for o, S in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(S, results[0][1])
    o_u, S_u = torch.empty_like(q), S0.clone()
    la.prefill(q, k, v, o_u, S_u, blk)
    torch.cuda.synchronize()
    d_o = (results[0][0].float() - o_u.float()).abs().max().item() / o_u.float().abs().max().item()
    d_s = (results[0][1] - S_u).abs().max().item() / S_u.abs().max().item()
    print(f"  cut vs uncut prefill: o {d_o:.3e} state {d_s:.3e}", flush=True)
    assert d_o <= TOL_BF16 and d_s <= 1e-4


def test_seqsplit_one_launch_waits_always_end():
    """The waits between the parts of a one-launch cut are bounded.  With the
    bound forced to zero ticks (LIN_ATTN_PART_WAIT_TICKS, which the library
    reads at each call), waits run out: the call still ends, and parts whose
    waits ran out give NaN rather than results from sums never written.  The
    next call, with the normal bound and the same workspace, is bitwise the
    normal result and leaves its flag words zero."""
    import os
    B, H, N, d, blk = 1, 8, 4096, 128, 64
    P = 16
    need = la.prefill_seqsplit_workspace(B, H, N, d, blk, torch.bfloat16)
    announce("prefill seqsplit one launch, zero-tick waits", B, H, N, d, blk)
    q, k, v = synth.prefill_inputs_device(45, B, H, N, d)
    S0 = torch.from_numpy(random_state(45, (B, H), d)).cuda()
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o_ref, S_ref = torch.empty_like(q), S0.clone()
    la.prefill_seqsplit(q, k, v, o_ref, S_ref, blk, ws)
    torch.cuda.synchronize()
    os.environ["LIN_ATTN_PART_WAIT_TICKS"] = "0"
    try:
        o, S = torch.empty_like(q), S0.clone()
        la.prefill_seqsplit(q, k, v, o, S, blk, ws)
        torch.cuda.synchronize()
    finally:
        del os.environ["LIN_ATTN_PART_WAIT_TICKS"]
    n_nan = int(torch.isnan(o.float()).sum())
    print(f"  zero-tick waits: {n_nan} of {o.numel()} outputs NaN", flush=True)
    assert n_nan > 0, "no wait ran out"
    o2, S2 = torch.empty_like(q), S0.clone()
    la.prefill_seqsplit(q, k, v, o2, S2, blk, ws)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(S2, S_ref)
    sums = (P - 1) * B * H * d * d * 4
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nsplit = 1
    while nsplit < 4 and B * H * P * nsplit < cus:
        nsplit *= 2
    flags = ws[2 * sums:].view(torch.int64).view(3, B * H, P, 4)
    used = torch.cat([flags[0, :, :P - 1, :nsplit].flatten(), flags[1, :, :, :nsplit].flatten(),
                      flags[2, :, :P - 1, :nsplit].flatten()])
    assert not torch.any(used), "flag words left set"


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


def test_workspace_queries_on_this_device():
    """The plans behind the workspace queries use the device's compute-unit
    count; on a 256-unit MI355X they give these sizes."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"sizes below are for 256 compute units, this device has {cus}")
    lib = la.library()
    q = lib.lin_attn_state_accumulate_split_workspace
    assert q(1, 64, 131072, 128, la.BF16) == 3 * 64 * 128 * 128 * 4  # 4 chunks of 32768 tokens
    assert q(4, 64, 32768, 128, la.BF16) == 0                         # 256 sequences: one chunk each
    assert q(1, 2, 255, 128, la.BF16) == 0                            # too short to split
    p = lib.lin_attn_prefill_seqsplit_workspace
    # 64 sequences of 131072 tokens: 4 parts of 32768, one launch: 3 * 64 part
    # sums and 3 * 64 start states of 64 KiB, then three flag arrays of
    # 64 * 4 * 4 words of 8 bytes
    assert p(1, 64, 131072, 128, 128, la.BF16) == 2 * 3 * 64 * 128 * 128 * 4 + 3 * 64 * 4 * 4 * 8
    # 4 sequences of 16384 tokens: 64 parts of 256, two launches (one state-pass
    # chunk each): 63 * 4 partial states + a copy of the 4 initial states
    assert p(1, 4, 16384, 128, 128, la.BF16) == (63 * 4 + 4) * 128 * 128 * 4
    assert p(4, 64, 32768, 128, 128, la.BF16) == 0
    assert p(1, 8, 4095, 128, 128, la.BF16) == 0       # indivisible: no cut
    # 8 sequences of 8192 tokens: 32 parts of 256, one launch
    assert p(1, 8, 8192, 128, 128, la.BF16) == 2 * 31 * 8 * 128 * 128 * 4 + 3 * 8 * 32 * 4 * 8
    assert p(1, 8, 510, 128, 128, la.BF16) == 0        # parts of 255 < 256: no cut
