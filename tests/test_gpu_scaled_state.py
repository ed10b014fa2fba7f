"""GPU parity of the narrow state formats (``lin_attn_decode_scaled``,
``lin_attn_decode`` with an FP8 state, ``lin_attn_prefill_scaled``) against
the fp64 oracle's stored-state model.

Storage model (the oracle's): entry x is stored as the bf16 or OCP FP8 E4M3
code of x / scale, rounded to nearest even (E4M3 clamped to +-448), and read
back as value(code) * scale.

Gates:
* stored codes equal the oracle's rounding of the exact (fp64) pre-store
  value, except where that value lies within the kernel's fp32 rounding of a
  midpoint between two codes; there the kernel may take either neighbour;
* outputs within 1e-5 of max|o| for fp32 I/O and 1e-2 for bf16 I/O (the
  gates of the fp32-state paths);
* exact-integer inputs whose every partial state is representable: bitwise;
* prefill with the carry rounded every block equals the same sequence
  prefilled one block per call with the state stored in between, bitwise.
"""
import numpy as np
import pytest
import torch

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import synth
from oracle import oracle

from gpu_helpers import announce, dev, host, rel_err

pytestmark = pytest.mark.gpu

FMTS = {"bf16": oracle.FMT_BF16, "e4m3": oracle.FMT_E4M3}
TOL_IO = {"fp32": 1e-5, "bf16": 1e-2}


def to_device_codes(codes: np.ndarray, fmt: str):
    if fmt == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def to_host_codes(t, fmt: str) -> np.ndarray:
    if fmt == "e4m3":
        return t.cpu().view(torch.uint8).numpy().copy()
    return t.cpu().view(torch.int16).numpy().view(np.uint16).copy()


def scales_for(lead, kind: str):
    """Per-sequence scales: powers of two, or (kind 'odd') values that are not."""
    n = int(np.prod(lead))
    base = np.array([0.5, 1.0, 2.0, 4.0, 0.25, 8.0, 16.0, 0.125], np.float32)
    if kind == "odd":
        base = np.array([3.0, 0.7, 1.3, 5.5, 0.3, 2.2, 9.0, 0.9], np.float32)
    return np.resize(base, n).reshape(lead).astype(np.float32)


def check_codes(got, x_exact, fmt: str, scale, rel_tol: float, abs_tol: float = 0.0):
    """Codes equal the oracle's rounding of x_exact, except next to a
    midpoint: where they differ, x_exact / scale lies within the tolerance of
    the midpoint of the two stored values."""
    f = FMTS[fmt]
    want = oracle.round_to_stored(x_exact, f, scale)
    diff = got != want
    if not diff.any():
        return 0
    sc = 1.0 if scale is None else np.asarray(scale, np.float64)[..., None, None]
    x = np.broadcast_to(np.asarray(x_exact, np.float64) / sc, got.shape)
    vg = oracle.stored_to_f64(got, f)
    vw = oracle.stored_to_f64(want, f)
    mid = (vg + vw) / 2
    ok = np.abs(x - mid) <= rel_tol * np.abs(x) + abs_tol
    bad = diff & ~ok
    assert not bad.any(), (f"{int(bad.sum())} of {int(diff.sum())} differing codes are not at a midpoint; first: "
                           f"x={x[bad][:3]}, gpu={vg[bad][:3]}, oracle={vw[bad][:3]}")
    return int(diff.sum())


# ---------------------------------------------------------------- decode ----

def decode_case(seed, B, H, d, io, fmt, scale):
    rng = np.random.default_rng([31, seed])
    lead = (B, H)
    sc = 1.0 if scale is None else scale[..., None, None].astype(np.float64)
    S0 = rng.standard_normal((*lead, d, d)) * 6.0 * sc
    codes = oracle.round_to_stored(S0, FMTS[fmt], scale)
    return codes


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
def test_decode_scaled_steps(d, io, fmt):
    """Four decode steps, each checked against the oracle from the codes the
    GPU holds before it (teacher forcing), with power-of-two scales."""
    announce("decode scaled steps", d, io, fmt)
    B, H = 2, 3
    scale = scales_for((B, H), "pow2")
    codes = decode_case(1, B, H, d, io, fmt, scale)
    Sd = to_device_codes(codes, fmt)
    scd = torch.from_numpy(scale).cuda()
    flips = 0
    for step in range(4):
        q, k, v = synth.decode_step_inputs(step, B, H, d, io)
        v = v * 4.0  # updates comparable to a stored-code step
        S_in = oracle.stored_to_f64(to_host_codes(Sd, fmt), FMTS[fmt], scale)
        o_ref, S_exact = oracle.recurrence(q[:, :, None], k[:, :, None], v[:, :, None], S_in)
        od = torch.empty_like(dev(q, io))
        la.decode(dev(q, io), dev(k, io), dev(v.astype(np.float32), io), od, Sd, state_scale=scd)
        torch.cuda.synchronize()
        flips += check_codes(to_host_codes(Sd, fmt), S_exact, fmt, scale, rel_tol=2.0 ** -22)
        e = rel_err(host(od), o_ref[:, :, 0])
        assert e <= TOL_IO[io], (step, e)
    print(f"  midpoint flips: {flips}")


@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
def test_decode_scaled_odd_scales(fmt):
    """Scales that are not powers of two: the scaling itself rounds in fp32,
    so the midpoint allowance widens to a few fp32 ulps."""
    announce("decode scaled odd scales", fmt)
    B, H, d = 2, 4, 128
    scale = scales_for((B, H), "odd")
    codes = decode_case(2, B, H, d, "fp32", fmt, scale)
    Sd = to_device_codes(codes, fmt)
    q, k, v = synth.decode_step_inputs(5, B, H, d, "fp32")
    S_in = oracle.stored_to_f64(codes, FMTS[fmt], scale)
    o_ref, S_exact = oracle.recurrence(q[:, :, None], k[:, :, None], v[:, :, None], S_in)
    od = torch.empty((B, H, d), device="cuda")
    la.decode(dev(q, "fp32"), dev(k, "fp32"), dev(v, "fp32"), od, Sd, state_scale=torch.from_numpy(scale).cuda())
    torch.cuda.synchronize()
    check_codes(to_host_codes(Sd, fmt), S_exact, fmt, scale, rel_tol=2.0 ** -19)
    assert rel_err(host(od), o_ref[:, :, 0]) <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
def test_decode_fp8_exact_integers(d):
    """Integer states within E4M3's exact range (|x| <= 16) and integer
    inputs: codes and outputs bitwise equal to the oracle over several steps;
    a power-of-two scale changes nothing but the stored units."""
    announce("decode fp8 exact integers", d)
    B, H, T = 2, 2, 6
    rng = np.random.default_rng([32, d])
    S = rng.integers(-3, 4, (B, H, d, d)).astype(np.float64)
    q, k, v = synth.integer_inputs(700 + d, B, H, T, d)
    for scale in (None, np.full((B, H), 0.5, np.float32)):
        codes = oracle.round_to_stored(S, oracle.FMT_E4M3, scale)
        ref_codes = codes.copy()
        o_ref = oracle.recurrence_stored_state(q, k, v, ref_codes, oracle.FMT_E4M3, scale=scale, block=1)
        bound = np.abs(S) + np.einsum("bhti,bhtj->bhij", np.abs(k), np.abs(v))
        assert bound.max() <= 16, "integer case leaves E4M3's exact range"
        Sd = to_device_codes(codes, "e4m3")
        scd = None if scale is None else torch.from_numpy(scale).cuda()
        for t in range(T):
            od = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
            la.decode(dev(q[:, :, t], "bf16"), dev(k[:, :, t], "bf16"), dev(v[:, :, t], "bf16"), od, Sd,
                      state_scale=scd)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(od), o_ref[:, :, t])
        np.testing.assert_array_equal(to_host_codes(Sd, "e4m3"), ref_codes)


def test_decode_fp8_unit_scale_is_plain_entry():
    """lin_attn_decode with an FP8 state is lin_attn_decode_scaled with unit
    scales, bit for bit; and a bf16 state with unit scales is the plain bf16
    decode."""
    announce("decode fp8 plain entry vs unit scales")
    B, H, d = 3, 4, 128
    for fmt in ("e4m3", "bf16"):
        codes = decode_case(3, B, H, d, "bf16", fmt, None)
        q, k, v = synth.decode_step_inputs(9, B, H, d, "bf16")
        A, Bst = to_device_codes(codes, fmt), to_device_codes(codes, fmt)
        oa = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
        ob = torch.empty_like(oa)
        la.decode(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), oa, A)
        la.decode(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), ob, Bst,
                  state_scale=torch.ones((B, H), device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
        np.testing.assert_array_equal(to_host_codes(A, fmt), to_host_codes(Bst, fmt))


def test_decode_fp8_many_steps_tracks_the_model():
    """64 free-running steps: the GPU's final state stays as close to the
    exact fp64 state as the oracle's storage model does (rounding decisions
    at midpoints may differ, the accumulated drift may not)."""
    announce("decode fp8 64 free-running steps")
    B, H, d, T = 2, 2, 128, 64
    scale = np.full((B, H), 0.25, np.float32)
    codes = decode_case(4, B, H, d, "bf16", "e4m3", scale)
    S0 = oracle.stored_to_f64(codes, oracle.FMT_E4M3, scale)
    q, k, v = synth.prefill_inputs(40, B, H, T, d, "bf16")
    model = codes.copy()
    oracle.recurrence_stored_state(q, k, v, model, oracle.FMT_E4M3, scale=scale, block=1)
    _, S_exact = oracle.recurrence(q, k, v, S0)
    Sd = to_device_codes(codes, "e4m3")
    scd = torch.from_numpy(scale).cuda()
    for t in range(T):
        od = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
        la.decode(dev(q[:, :, t], "bf16"), dev(k[:, :, t], "bf16"), dev(v[:, :, t], "bf16"), od, Sd, state_scale=scd)
    torch.cuda.synchronize()
    S_gpu = oracle.stored_to_f64(to_host_codes(Sd, "e4m3"), oracle.FMT_E4M3, scale)
    S_model = oracle.stored_to_f64(model, oracle.FMT_E4M3, scale)
    e_gpu, e_model = rel_err(S_gpu, S_exact), rel_err(S_model, S_exact)
    mism = float(np.mean(to_host_codes(Sd, "e4m3") != model))
    print(f"  drift gpu={e_gpu:.3e} model={e_model:.3e}; codes differing from the model: {mism:.2%}")
    assert e_gpu <= 1.25 * e_model + 1e-6
    assert mism <= 0.02


# --------------------------------------------------------------- prefill ----

def run_prefill_scaled(q, k, v, codes, fmt, scale, block, round_carry):
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    od = torch.empty_like(qd)
    Sd = to_device_codes(codes, fmt)
    scd = None if scale is None else torch.from_numpy(np.ascontiguousarray(scale, np.float32)).cuda()
    la.prefill_scaled(qd, kd, vd, od, Sd, block, state_scale=scd, round_carry=round_carry)
    torch.cuda.synchronize()
    return host(od), to_host_codes(Sd, fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
@pytest.mark.parametrize("d,N,block", [(128, 1, 64), (128, 77, 16), (128, 300, 128), (64, 129, 32), (64, 400, 64)])
def test_prefill_scaled_exact_integers(fmt, d, N, block):
    """Integer inputs and states inside the format's exact range: outputs and
    stored state bitwise equal to the oracle, with and without carry
    rounding (nothing rounds, so both equal the fp64 recurrence)."""
    announce("prefill scaled exact integers", fmt, d, N, block)
    B, H = 1, 3
    q, k, v = synth.integer_inputs(800 + d + N, B, H, N, d)
    rng = np.random.default_rng([33, d, N])
    S0 = rng.integers(-3, 4, (B, H, d, d)).astype(np.float64)
    bound = np.abs(S0) + np.einsum("bhti,bhtj->bhij", np.abs(k), np.abs(v))
    assert bound.max() <= (16 if fmt == "e4m3" else 256), "integer case leaves the exact range"
    o_ref, S_ref = oracle.recurrence(q, k, v, S0)
    assert np.abs(o_ref).max() <= 256, "integer outputs leave bf16's exact range"
    for rc in (False, True):
        o, codes = run_prefill_scaled(q, k, v, oracle.round_to_stored(S0, FMTS[fmt]), fmt, None, block, rc)
        np.testing.assert_array_equal(o, o_ref)
        np.testing.assert_array_equal(oracle.stored_to_f64(codes, FMTS[fmt]), S_ref)


@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
@pytest.mark.parametrize("d,N,block,H", [(128, 1000, 128, 3), (128, 333, 64, 70), (64, 517, 96, 4),
                                          (128, 130, 128, 256)])
def test_prefill_scaled_no_carry_rounding(fmt, d, N, block, H):
    """round_carry = 0: outputs bit-identical to the fp32-state prefill from
    the widened S_0; the stored S_N is the oracle's rounding of the exact
    S_N within the fp32 accumulation's reach of a midpoint; outputs within
    the bf16 gate of the oracle."""
    announce("prefill scaled, carry in fp32", fmt, d, N, block, H)
    B = 1
    q, k, v = synth.prefill_inputs(41, B, H, N, d, "bf16")
    scale = scales_for((B, H), "pow2")
    rng = np.random.default_rng([34, d])
    codes = oracle.round_to_stored(rng.standard_normal((B, H, d, d)) * 4 * scale[..., None, None], FMTS[fmt], scale)
    S0 = oracle.stored_to_f64(codes, FMTS[fmt], scale)
    o, got = run_prefill_scaled(q, k, v, codes, fmt, scale, block, False)
    # the same kernel arithmetic with an fp32 state
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o32 = torch.empty_like(qd)
    S32 = torch.from_numpy(S0.astype(np.float32)).cuda()
    la.prefill(qd, kd, vd, o32, S32, block)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o, host(o32))
    o_ref, S_exact = oracle.recurrence(q, k, v, S0)
    assert rel_err(o, o_ref) <= 1e-2
    n = check_codes(got, S_exact, fmt, scale, rel_tol=0.0,
                    abs_tol=2e-6 * float(np.max(np.abs(S_exact / scale[..., None, None]))))
    print(f"  midpoint flips: {n}")


@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
@pytest.mark.parametrize("d,N,block,H", [(128, 1000, 128, 2), (128, 700, 64, 66), (64, 450, 32, 3)])
def test_prefill_scaled_carry_rounding(fmt, d, N, block, H):
    """round_carry = 1.  (a) The whole sequence in one call equals the
    sequence prefilled one block per call with the state stored in between,
    bit for bit.  (b) Each of those one-block calls matches the oracle from
    the codes it started from: codes up to midpoints, outputs to 1e-2."""
    announce("prefill scaled, carry rounded every block", fmt, d, N, block, H)
    B = 1
    q, k, v = synth.prefill_inputs(42, B, H, N, d, "bf16")
    scale = scales_for((B, H), "pow2")
    rng = np.random.default_rng([35, d])
    codes0 = oracle.round_to_stored(rng.standard_normal((B, H, d, d)) * 4 * scale[..., None, None], FMTS[fmt], scale)
    o_full, codes_full = run_prefill_scaled(q, k, v, codes0, fmt, scale, block, True)
    codes = codes0
    outs = []
    flips = 0
    for t0 in range(0, N, block):
        sl = slice(t0, min(t0 + block, N))
        o_b, nxt = run_prefill_scaled(q[:, :, sl], k[:, :, sl], v[:, :, sl], codes, fmt, scale, block, True)
        S_in = oracle.stored_to_f64(codes, FMTS[fmt], scale)
        o_ref, S_exact = oracle.recurrence(q[:, :, sl], k[:, :, sl], v[:, :, sl], S_in)
        assert rel_err(o_b, o_ref) <= 1e-2, t0
        flips += check_codes(nxt, S_exact, fmt, scale, rel_tol=0.0,
                             abs_tol=2e-6 * float(np.max(np.abs(S_exact / scale[..., None, None]))))
        outs.append(o_b)
        codes = nxt
    np.testing.assert_array_equal(codes_full, codes)
    np.testing.assert_array_equal(o_full, np.concatenate(outs, axis=2))
    print(f"  blocks: {len(outs)}, midpoint flips: {flips}")


# ------------------------------------------------ verify / commit drafts ----

@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
@pytest.mark.parametrize("d,T,io", [(128, 4, "bf16"), (128, 16, "fp32"), (64, 7, "bf16"), (64, 1, "fp32")])
def test_verify_scaled(fmt, d, T, io):
    """Draft outputs from a narrow stored state with per-sequence scales
    equal the oracle run from the widened state; the state is untouched."""
    announce("verify scaled", fmt, d, T, io)
    B, H = 2, 3
    scale = scales_for((B, H), "pow2")
    codes = decode_case(20 + T, B, H, d, io, fmt, scale)
    q, k, v = synth.prefill_inputs(80 + T, B, H, T, d, io)
    o_ref, _ = oracle.recurrence(q, k, v, oracle.stored_to_f64(codes, FMTS[fmt], scale))
    Sd = to_device_codes(codes, fmt)
    od = torch.empty((B, H, T, d), dtype=dev(q, io).dtype, device="cuda")
    la.decode_verify(dev(q, io), dev(k, io), dev(v, io), od, Sd, state_scale=torch.from_numpy(scale).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host_codes(Sd, fmt), codes)
    e = rel_err(host(od), o_ref)
    print(f"  rel err o={e:.3e}")
    assert e <= TOL_IO[io]


@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
@pytest.mark.parametrize("d,T", [(128, 4), (64, 16)])
def test_commit_scaled(fmt, d, T):
    """Commit of per-sequence accepted counts (0 .. T, clamped): the stored
    state is the oracle's single rounding of the widened state plus the
    accepted drafts, up to fp32 midpoint ties; accepting 0 leaves it
    bit-identical."""
    announce("commit scaled", fmt, d, T)
    B, H = 4, 2
    scale = scales_for((B, H), "pow2")
    codes = decode_case(30 + T, B, H, d, "bf16", fmt, scale)
    _, k, v = synth.prefill_inputs(90 + T, B, H, T, d, "bf16")
    v = v * 4.0  # updates comparable to a stored-code step
    accept = np.array([0, 1, T, T + 5], np.int32)
    Sd = to_device_codes(codes, fmt)
    la.decode_commit(dev(k, "bf16"), dev(v, "bf16"), Sd, torch.from_numpy(accept).cuda(),
                     state_scale=torch.from_numpy(scale).cuda())
    torch.cuda.synchronize()
    got = to_host_codes(Sd, fmt)
    S_in = oracle.stored_to_f64(codes, FMTS[fmt], scale)
    for b in range(B):
        a_b = int(min(max(accept[b], 0), T))
        if a_b == 0:
            np.testing.assert_array_equal(got[b], codes[b])
            continue
        S_exact = oracle.state_after(k[b, :, :a_b], v[b, :, :a_b], S_in[b])
        # fp32 sums of up to 16 terms: a few fp32 ulps from the exact value
        n = check_codes(got[b], S_exact, fmt, scale[b], rel_tol=2.0 ** -19,
                        abs_tol=1e-6 * float(np.max(np.abs(S_exact / scale[b][:, None, None]))))
        print(f"  batch {b}: accepted {a_b}, midpoint flips {n}")


def test_verify_commit_fp8_unit_scale_is_plain_entry():
    """The unscaled verify and commit with an FP8 state are the scaled ones
    with unit scales, bit for bit."""
    announce("verify/commit fp8 plain entry vs unit scales")
    B, H, T, d = 2, 3, 5, 128
    codes = decode_case(40, B, H, d, "bf16", "e4m3", None)
    q, k, v = synth.prefill_inputs(95, B, H, T, d, "bf16")
    ones = torch.ones((B, H), device="cuda")
    outs, states = [], []
    for sc in (None, ones):
        Sd = to_device_codes(codes, "e4m3")
        od = torch.empty((B, H, T, d), dtype=torch.bfloat16, device="cuda")
        la.decode_verify(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), od, Sd, state_scale=sc)
        la.decode_commit(dev(k, "bf16"), dev(v, "bf16"), Sd, state_scale=sc)
        torch.cuda.synchronize()
        outs.append(od.view(torch.int16).cpu())
        states.append(to_host_codes(Sd, "e4m3"))
    assert torch.equal(outs[0], outs[1])
    np.testing.assert_array_equal(states[0], states[1])


def test_commit_fp8_exact_integers():
    """Integer states and drafts within E4M3's exact range: the committed
    state equals the oracle's bitwise, for every accepted count."""
    announce("commit fp8 exact integers")
    B, H, T, d = 3, 2, 6, 128
    rng = np.random.default_rng(77)
    S = rng.integers(-3, 4, (B, H, d, d)).astype(np.float64)
    _, k, v = synth.integer_inputs(777, B, H, T, d)
    assert (np.abs(S) + np.einsum("bhti,bhtj->bhij", np.abs(k), np.abs(v))).max() <= 16
    accept = np.array([2, 0, 6], np.int32)
    Sd = to_device_codes(oracle.round_to_stored(S, oracle.FMT_E4M3), "e4m3")
    la.decode_commit(dev(k, "bf16"), dev(v, "bf16"), Sd, torch.from_numpy(accept).cuda())
    torch.cuda.synchronize()
    got = oracle.stored_to_f64(to_host_codes(Sd, "e4m3"), oracle.FMT_E4M3)
    for b in range(B):
        np.testing.assert_array_equal(got[b], oracle.state_after(k[b, :, :accept[b]], v[b, :, :accept[b]], S[b]))


@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
@pytest.mark.parametrize("d", [128, 64])
def test_decode_and_commit_odd_head_count(fmt, d):
    """Seven sequences: decode and commit give two waves to each head (two
    heads per workgroup), so the last workgroup holds one head and a pair of
    idle waves.  Stored codes against the oracle's rounding, as above."""
    announce("decode / commit odd head count", fmt, d)
    B, H, T = 1, 7, 3
    scale = scales_for((B, H), "pow2")
    codes = decode_case(40, B, H, d, "bf16", fmt, scale)
    scd = torch.from_numpy(scale).cuda()
    # one decode step
    Sd = to_device_codes(codes, fmt)
    q, k, v = synth.decode_step_inputs(9, B, H, d, "bf16")
    S_in = oracle.stored_to_f64(codes, FMTS[fmt], scale)
    o_ref, S_exact = oracle.recurrence(q[:, :, None], k[:, :, None], v[:, :, None], S_in)
    od = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    la.decode(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), od, Sd, state_scale=scd)
    torch.cuda.synchronize()
    check_codes(to_host_codes(Sd, fmt), S_exact, fmt, scale, rel_tol=2.0 ** -22)
    assert rel_err(host(od), o_ref[:, :, 0]) <= TOL_IO["bf16"]
    # a commit of all T drafts on the same codes
    Sc = to_device_codes(codes, fmt)
    _, kc, vc = synth.prefill_inputs(91, B, H, T, d, "bf16")
    la.decode_commit(dev(kc, "bf16"), dev(vc, "bf16"), Sc, state_scale=scd)
    torch.cuda.synchronize()
    got = to_host_codes(Sc, fmt)
    for h in range(H):
        S_h = oracle.state_after(kc[0, h], vc[0, h], S_in[0, h])
        check_codes(got[0, h], S_h, fmt, scale[0, h], rel_tol=2.0 ** -19,
                    abs_tol=1e-6 * float(np.max(np.abs(S_h / scale[0, h]))))
