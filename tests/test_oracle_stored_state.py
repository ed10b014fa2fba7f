"""Pins of the oracle's low-precision state storage against facts that do not
come from the oracle.

The model pinned: a state rewritten again and again in a narrow format
("ノーフリーランチ：MiniMax M2が高効率アテンション機構を解体" (winzheng.jp),
section "推論システム統合の課題": FP8 or other low-precision storage of the
state accumulates rounding error), stored every `block` tokens in bf16 or in
OCP FP8 E4M3 with a per-head scale, the tokens in between running through the
exact recurrence from the widened store.

Pins used:
* the E4M3 rounding and widening against torch's ``float8_e4m3fn``
  conversion (an independent library implementation of the same format) on
  every value it represents in range, with exact ties, and against the
  format's definition on doubles (half-ulp bound, ties to even, saturation);
* exact-integer inputs whose every partial state is representable: no
  rounding happens, so the result equals the fp64 recurrence;
* block = 1 with bf16 equals the separately written bf16 decode-step model;
* the block composition built from the pinned recurrence and the pinned
  roundings, including a ragged last block;
* the exact power-of-two scale invariance;
* planted mistakes in copies of the oracle that the pins must reject.
"""
import numpy as np
import pytest
import torch

from oracle import oracle

E4M3 = oracle.FMT_E4M3
BF16 = oracle.FMT_BF16


def torch_e4m3_codes(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_grid() -> np.ndarray:
    """Every finite non-negative E4M3 value, by torch's widening."""
    vals = torch.arange(0, 128, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return np.unique(vals[np.isfinite(vals)].astype(np.float64))


# ------------------------------------------------------------ E4M3 pins ----

def check_widen(lib=oracle):
    codes = np.arange(256, dtype=np.uint8)
    got = lib.e4m3_codes_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def check_round_vs_torch(lib=oracle):
    rng = np.random.default_rng(11)
    grid = e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2  # exact ties, all representable in float32
    x = np.concatenate([
        rng.uniform(-460, 460, 50000),
        rng.standard_normal(50000) * 2.0 ** rng.integers(-14, 8, 50000),
        grid, -grid, mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(0)), np.nextafter(mids.astype(np.float32), np.float32(1e9)),
        [0.0, -0.0, 2.0 ** -12, 2.0 ** -10, 3 * 2.0 ** -11, 463.99, -463.99, 464.0, -464.0],
    ]).astype(np.float32)
    x = x[np.abs(x) <= 464]  # torch turns values beyond 464 into NaN; the oracle clamps them
    got = lib.round_e4m3_codes(x.astype(np.float64))
    ref = torch_e4m3_codes(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


def check_round_definition(lib=oracle):
    """On doubles: the result is an E4M3 value within half a spacing, ties go
    to the even code, beyond the largest finite value it saturates."""
    rng = np.random.default_rng(12)
    grid = e4m3_grid()
    x = rng.uniform(2.0 ** -9, 447.0, 20000) * rng.choice([-1.0, 1.0], 20000)
    c = lib.round_e4m3_codes(x)
    r = lib.e4m3_codes_to_f64(c)
    a = np.abs(x)
    idx = np.clip(np.searchsorted(grid, a), 1, grid.size - 1)
    lo, hi = grid[idx - 1], grid[idx]
    assert np.all(np.abs(a - np.abs(r)) <= (hi - lo) / 2 * (1 + 1e-15))
    assert np.all(np.signbit(r) == np.signbit(x))
    mids = (grid[:-1] + grid[1:]) / 2
    assert np.all(lib.round_e4m3_codes(mids) % 2 == 0)
    big = np.array([448.0, 448.5, 464.0, 465.0, 480.0, 1e30, np.inf])
    assert np.all(lib.round_e4m3_codes(big) == 0x7E)
    assert np.all(lib.round_e4m3_codes(-big) == 0xFE)
    assert np.isnan(lib.e4m3_codes_to_f64(lib.round_e4m3_codes(np.array([np.nan])))[0])
    # the subnormal range: multiples of 2^-9 below 2^-6 are exact
    sub = np.arange(0, 9) * 2.0 ** -9
    assert np.array_equal(lib.e4m3_codes_to_f64(lib.round_e4m3_codes(sub)), sub)
    assert lib.round_e4m3_codes(np.array([2.0 ** -10]))[0] == 0  # tie with 0: even
    assert lib.round_e4m3_codes(np.array([3 * 2.0 ** -10]))[0] == 2  # tie 1 / 2: even


E4M3_PINS = [check_widen, check_round_vs_torch, check_round_definition]


@pytest.mark.parametrize("pin", E4M3_PINS, ids=lambda f: f.__name__)
def test_e4m3_pin(pin):
    pin()


# ------------------------------------------------ stored-state model pins ----

def int_case(seed, lead, N, d, s_range, kv_range=1):
    rng = np.random.default_rng(seed)
    q = rng.integers(-2, 3, (*lead, N, d)).astype(np.float32)
    k = rng.integers(-kv_range, kv_range + 1, (*lead, N, d)).astype(np.float32)
    v = rng.integers(-kv_range, kv_range + 1, (*lead, N, d)).astype(np.float32)
    S0 = rng.integers(-s_range, s_range + 1, (*lead, d, d)).astype(np.float64)
    return q, k, v, S0


def check_exact_integers(lib=oracle):
    """Every partial state stays on the format's integer grid: no rounding,
    so outputs and final state equal the fp64 recurrence for any block."""
    for fmt, s_range, N in ((E4M3, 3, 8), (BF16, 100, 40)):
        q, k, v, S0 = int_case(21 + fmt, (2, 3), N, 4, s_range)
        # |S_t| <= s_range + t for entries of k, v in {-1, 0, 1}: E4M3 holds all
        # integers up to 16, bf16 up to 256
        o_ref, S_ref = oracle.recurrence(q, k, v, S0)
        for block in (1, 3, N, N + 5):
            codes = lib.round_to_stored(S0, fmt)
            o = lib.recurrence_stored_state(q, k, v, codes, fmt, block=block)
            assert np.array_equal(o, o_ref), (fmt, block)
            assert np.array_equal(lib.stored_to_f64(codes, fmt), S_ref), (fmt, block)


def check_single_store(lib=oracle):
    """block >= N: outputs are the fp64 recurrence from the widened S_0 and
    the state is stored once, rounded from the exact S_N."""
    rng = np.random.default_rng(22)
    for fmt in (BF16, E4M3):
        q = rng.standard_normal((2, 17, 8)).astype(np.float32)
        k = rng.standard_normal((2, 17, 8)).astype(np.float32)
        v = rng.standard_normal((2, 17, 8)).astype(np.float32)
        codes = lib.round_to_stored(rng.standard_normal((2, 8, 8)) * 4, fmt)
        S0 = lib.stored_to_f64(codes, fmt)
        o_ref, S_ref = oracle.recurrence(q, k, v, S0)
        o = lib.recurrence_stored_state(q, k, v, codes, fmt, block=17)
        assert np.array_equal(o, o_ref)
        assert np.array_equal(codes, lib.round_to_stored(S_ref, fmt))


def check_bf16_decode_steps(lib=oracle):
    """block = 1 in bf16 is the separately written bf16 decode-step model."""
    rng = np.random.default_rng(23)
    H, N, d = 3, 6, 8
    q = rng.standard_normal((H, N, d)).astype(np.float32)
    k = rng.standard_normal((H, N, d)).astype(np.float32)
    v = rng.standard_normal((H, N, d)).astype(np.float32)
    S0 = rng.standard_normal((H, d, d)) * 3
    codes = oracle.round_bf16_bits(S0)
    steps = codes.copy()
    o = lib.recurrence_stored_state(q, k, v, codes, BF16, block=1)
    for t in range(N):
        ot = oracle.decode_step_bf16_state(q[:, t], k[:, t], v[:, t], steps)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(codes, steps)


def check_block_composition(lib=oracle):
    """Ragged block boundaries: each block runs the pinned recurrence from the
    widened store and is rounded by the pinned conversion."""
    rng = np.random.default_rng(24)
    H, N, d, block = 2, 23, 8, 5
    for fmt, sc in ((BF16, None), (E4M3, np.array([0.25, 2.0], np.float32))):
        q = rng.standard_normal((H, N, d)).astype(np.float32)
        k = rng.standard_normal((H, N, d)).astype(np.float32)
        v = rng.standard_normal((H, N, d)).astype(np.float32)
        codes = lib.round_to_stored(rng.standard_normal((H, d, d)), fmt, sc)
        ref_codes = codes.copy()
        o = lib.recurrence_stored_state(q, k, v, codes, fmt, scale=sc, block=block)
        o_ref = np.empty_like(o)
        for t0 in range(0, N, block):
            S = oracle.stored_to_f64(ref_codes, fmt, sc)
            o_ref[:, t0:t0 + block], S = oracle.recurrence(q[:, t0:t0 + block], k[:, t0:t0 + block],
                                                           v[:, t0:t0 + block], S)
            ref_codes = oracle.round_to_stored(S, fmt, sc)
        assert np.array_equal(o, o_ref), fmt
        assert np.array_equal(codes, ref_codes), fmt


def check_scale_invariance(lib=oracle):
    """Multiplying v and the scale by 2^m multiplies outputs by 2^m and leaves
    every code unchanged (exact in binary floating point)."""
    rng = np.random.default_rng(25)
    H, N, d = 2, 30, 8
    q = rng.standard_normal((H, N, d)).astype(np.float32)
    k = rng.standard_normal((H, N, d)).astype(np.float32)
    v = rng.standard_normal((H, N, d)).astype(np.float32)
    for fmt in (BF16, E4M3):
        c1 = lib.round_to_stored(rng.standard_normal((H, d, d)), fmt)
        c2 = c1.copy()
        o1 = lib.recurrence_stored_state(q, k, v, c1, fmt, scale=None, block=4)
        o2 = lib.recurrence_stored_state(q, k, (v * 8).astype(np.float32), c2, fmt,
                                         scale=np.full(H, 8.0, np.float32), block=4)
        assert np.array_equal(o2, o1 * 8)
        assert np.array_equal(c1, c2)
        assert np.array_equal(lib.stored_to_f64(c2, fmt, np.full(H, 8.0, np.float32)), lib.stored_to_f64(c1, fmt) * 8)


STORED_PINS = [check_exact_integers, check_single_store, check_bf16_decode_steps, check_block_composition,
               check_scale_invariance]


@pytest.mark.parametrize("pin", STORED_PINS, ids=lambda f: f.__name__)
def test_stored_state_pin(pin):
    pin()


def test_stored_state_rejects_bad_arguments():
    q = np.zeros((1, 2, 4), np.float32)
    codes = np.zeros((1, 4, 4), np.uint8)
    with pytest.raises(RuntimeError):
        oracle.recurrence_stored_state(q, q, q, codes, E4M3, block=0)
    with pytest.raises(RuntimeError):
        oracle.recurrence_stored_state(q, q, q, codes, E4M3, scale=np.zeros(1, np.float32))
    with pytest.raises(TypeError):
        oracle.recurrence_stored_state(q, q, q, codes, BF16)


def test_e4m3_storage_loses_small_updates():
    """The hazard itself: once the state is 16 or more times the per-token
    update, E4M3 storage (3 fraction bits) rounds every update away, while
    the exact state keeps growing."""
    d, N = 4, 64
    q = np.ones((1, N, d), np.float32)
    k = np.full((1, N, d), 0.5, np.float32)
    v = np.full((1, N, d), 0.5, np.float32)  # each token adds 0.25 to every entry
    codes = oracle.round_e4m3_codes(np.full((1, d, d), 8.0))  # 8 = 32 updates
    oracle.recurrence_stored_state(q, k, v, codes, E4M3, block=1)
    assert np.all(oracle.e4m3_codes_to_f64(codes) == 8.0)  # 8.25 rounds back to 8
    codes = oracle.round_e4m3_codes(np.full((1, d, d), 8.0))
    oracle.recurrence_stored_state(q, k, v, codes, E4M3, block=N)
    assert np.all(oracle.e4m3_codes_to_f64(codes) == 24.0)  # 8 + 64 * 0.25


# --------------------------------------------- planted mistakes (CPU) ----

STORED_MUTANTS = {
    "carry_not_rewidened": ("      double_to_stored(codes, i, fmt, work[i], scale);\n      work[i] = stored_to_double(codes, i, fmt, scale);",
                            "      double_to_stored(codes, i, fmt, work[i], scale);"),
    "scale_multiplied_on_store": ("double_to_e4m3_rne_sat(x / scale)", "double_to_e4m3_rne_sat(x * scale)"),
    "bias_off_by_one": ("return (uint8_t)(sign | ((unb + 7) << 3) | (mant - 8));",
                        "return (uint8_t)(sign | ((unb + 8) << 3) | (mant - 8));"),
    "subnormal_floor": ("if (unb < -6) unb = -6;     /* subnormals share the smallest exponent */",
                        "if (unb < -7) unb = -7;     /* subnormals share the smallest exponent */"),
    "truncating_round": ("double r = rint(ldexp(a, 3 - unb)); /* grid step 2^(unb-3) */",
                         "double r = floor(ldexp(a, 3 - unb)); /* grid step 2^(unb-3) */"),
    "widen_subnormal_scale": ("else if (e == 0) y = ldexp((double)f, -9);", "else if (e == 0) y = ldexp((double)f, -10);"),
    "ragged_tail_dropped": ("for (int64_t t0 = 0; t0 < N; t0 += block) {",
                            "for (int64_t t0 = 0; t0 + block <= N; t0 += block) {"),
}


@pytest.mark.parametrize("name", sorted(STORED_MUTANTS))
def test_stored_pins_reject_planted_mistakes(name, tmp_path):
    old, new = STORED_MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation target for {name} not found verbatim in the oracle"
    variant = oracle.compile_variant(src.replace(old, new), str(tmp_path / f"mut_{name}.so"))
    caught = []
    for pin in E4M3_PINS + STORED_PINS:
        try:
            pin(variant)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the planted mistake {name}"
