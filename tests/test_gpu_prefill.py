"""GPU parity of the chunked prefill (bf16 MFMA path and fp32 path) against
the fp64 oracle, element by element, plus the invariants the method implies.

Gates: max|gpu - oracle| / max|oracle| <= 1e-2 for bf16 inputs with an fp32
state, <= 1e-4 for fp32 inputs; exact equality for exact-integer inputs.
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


def integer_case(seed, B, H, N, d):
    q, k, v = synth.integer_inputs(seed, B, H, N, d)
    rng = np.random.default_rng([3, seed])
    S0 = rng.integers(-2, 3, size=(B, H, d, d)).astype(np.float32)
    # every partial sum the kernel can form is bounded by these sums of absolute
    # values; keep them within the integers bf16 represents exactly (|x| <= 256)
    abs_s = np.abs(S0).astype(np.float64) + np.einsum("bhti,bhtj->bhij", np.abs(k), np.abs(v))
    abs_p = np.einsum("bhti,bhsi->bhts", np.abs(q), np.abs(k))
    abs_o = np.einsum("bhts,bhsj->bhtj", abs_p, np.abs(v)) + np.einsum("bhti,bhij->bhtj", np.abs(q), abs_s)
    assert abs_s.max() <= 256 and abs_o.max() <= 256, "integer case leaves the exact range"
    return q, k, v, S0


@pytest.mark.parametrize("d,block,N,split", [
    (128, 64, 300, 1), (128, 128, 300, 1), (128, 16, 77, 1), (128, 48, 200, 1), (128, 96, 250, 1),
    (128, 128, 257, 2), (128, 64, 190, 4), (128, 112, 129, 4),
    (64, 64, 300, 1), (64, 128, 600, 1), (64, 32, 95, 2), (64, 112, 430, 2), (64, 80, 333, 1),
])
def test_prefill_bf16_exact_integers(d, block, N, split):
    announce("prefill bf16 exact-integer", d, block, N, split)
    q, k, v, S0 = integer_case(1000 + d + block + N, 1, 2, N, d)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    o, S = gpu_prefill(q, k, v, S0, block, "bf16", split)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(S, S_ref)


@pytest.mark.parametrize("d,block,N", [(128, 64, 150), (64, 128, 300), (128, 16, 40)])
def test_prefill_f32_exact_integers(d, block, N):
    announce("prefill fp32 exact-integer", d, block, N)
    q, k, v, S0 = integer_case(2000 + d + block + N, 1, 2, N, d)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    o, S = gpu_prefill(q, k, v, S0, block, "fp32")
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(S, S_ref)


@pytest.mark.parametrize("B,H,N,d,block,split", [
    (1, 3, 1000, 128, 64, 0), (2, 2, 777, 128, 128, 1), (1, 2, 500, 128, 128, 2),
    (1, 2, 500, 128, 128, 4), (2, 3, 700, 64, 64, 1), (1, 2, 513, 64, 128, 2), (1, 2, 300, 128, 96, 0),
    (1, 1, 33, 128, 16, 1), (1, 2, 250, 128, 48, 1), (1, 1, 1, 128, 128, 1), (1, 2, 5, 64, 64, 0),
])
def test_prefill_bf16_random(B, H, N, d, block, split):
    announce("prefill bf16 random", B, H, N, d, block, split)
    q, k, v = synth.prefill_inputs(10, B, H, N, d, "bf16")
    S0 = random_state(N + d, (B, H), d, scale=4.0)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    o, S = gpu_prefill(q, k, v, S0, block, "bf16", split)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    print(f"  rel err o={eo:.3e} state={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_prefill_f32_workload_small():
    """The small fp32 workload: 1 head, N=256, d=64, block 64, zero state."""
    announce("prefill fp32 B1 H1 N256 d64 blk64")
    q, k, v = synth.prefill_inputs(1, 1, 1, 256, 64, "fp32")
    S0 = np.zeros((1, 1, 64, 64), np.float32)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    o, S = gpu_prefill(q, k, v, S0, 64, "fp32")
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    print(f"  rel err o={eo:.3e} state={es:.3e}")
    assert eo <= TOL_F32 and es <= TOL_F32


@pytest.mark.parametrize("B,H,N,d,block", [(1, 2, 300, 128, 64), (2, 1, 257, 64, 128), (1, 1, 70, 128, 16),
                                           (1, 2, 100, 64, 48)])
def test_prefill_f32_random(B, H, N, d, block):
    announce("prefill fp32 random", B, H, N, d, block)
    q, k, v = synth.prefill_inputs(11, B, H, N, d, "fp32")
    S0 = random_state(N, (B, H), d)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    o, S = gpu_prefill(q, k, v, S0, block, "fp32")
    assert rel_err(o, o_ref) <= TOL_F32 and rel_err(S, S_ref) <= TOL_F32


def test_prefill_empty_is_noop():
    announce("prefill N=0 no-op")
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    S = torch.randn((1, 2, 128, 128), device="cuda")
    S_before = S.clone()
    la.prefill(q, q, q, q.clone(), S, 64)
    torch.cuda.synchronize()
    assert torch.equal(S, S_before)


def test_prefill_deterministic_and_split_invariant():
    """Repeated runs are bitwise identical, and so are all value-column
    splits: each output column sees the same products in the same order."""
    announce("prefill determinism / split invariance")
    B, H, N, d = 1, 4, 700, 128
    q, k, v = synth.prefill_inputs(12, B, H, N, d, "bf16")
    S0 = random_state(5, (B, H), d)
    runs = [gpu_prefill(q, k, v, S0, 128, "bf16", s) for s in (1, 1, 2, 4)]
    for o, S in runs[1:]:
        np.testing.assert_array_equal(o, runs[0][0])
        np.testing.assert_array_equal(S, runs[0][1])


@pytest.mark.parametrize("block,n_first", [(64, 256), (128, 384), (64, 100)])
def test_prefill_continuation(block, n_first):
    """prefill(x[:n]) then prefill(x[n:]) from the carried state equals
    prefill(x): bitwise when n is a multiple of the block (same tiles), within
    tolerance otherwise."""
    announce("prefill continuation", block, n_first)
    B, H, N, d = 1, 2, 640, 128
    q, k, v = synth.prefill_inputs(13, B, H, N, d, "bf16")
    S0 = random_state(6, (B, H), d)
    o_all, S_all = gpu_prefill(q, k, v, S0, block, "bf16", 1)
    o1, S1 = gpu_prefill(q[:, :, :n_first], k[:, :, :n_first], v[:, :, :n_first], S0, block, "bf16", 1)
    o2, S2 = gpu_prefill(q[:, :, n_first:], k[:, :, n_first:], v[:, :, n_first:], S1.astype(np.float32),
                         block, "bf16", 1)
    o_cat = np.concatenate([o1, o2], axis=2)
    if n_first % block == 0:
        np.testing.assert_array_equal(o_cat, o_all)
        np.testing.assert_array_equal(S2, S_all)
    else:
        assert rel_err(o_cat, o_all) <= TOL_BF16 and rel_err(S2, S_all) <= TOL_BF16


def test_prefill_block_independence():
    """The block size changes rounding only: every block size agrees with the
    oracle, hence with every other block size, within the gate."""
    announce("prefill block independence")
    B, H, N, d = 1, 2, 400, 128
    q, k, v = synth.prefill_inputs(14, B, H, N, d, "bf16")
    S0 = random_state(7, (B, H), d)
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    for block in (16, 32, 64, 80, 128):
        o, S = gpu_prefill(q, k, v, S0, block, "bf16")
        assert rel_err(o, o_ref) <= TOL_BF16 and rel_err(S, S_ref) <= TOL_BF16, block


def test_binding_rejects_mismatched_tensors():
    announce("binding checks")
    q = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    S = torch.zeros((1, 1, 128, 128), device="cuda")
    with pytest.raises(TypeError):
        la.prefill(q, q, q.float(), q.clone(), S, 64)
    with pytest.raises(ValueError):
        la.prefill(q, q, q, q.clone(), S[:, :, :64], 64)
    with pytest.raises(la.LinAttnError) as e:
        la.prefill(q, q, q, q.clone(), S, 40)
    assert e.value.code == la.EUNSUPPORTED
