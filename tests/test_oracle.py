"""Pins of the fp64 oracle against facts that do not come from the oracle.

The definition being pinned: causal linear attention through the recurrence
S_t = S_{t-1} + k_t v_t^T, o_t = q_t^T S_t ("MiniMax-M1で理解する：大規模言語
モデルのコンテキスト長限界を突破する革新的アーキテクチャ", zenn.dev, section
"線形アテンションの数学的基礎", recurrence equations; phi = identity), whose
tiled form ("Почему M2 в итоге стала моделью с полным вниманием?",
ai.flicky.cc, section 1, glossary entry "Lightning Attention") is an exact
re-association.

Pins used (none of them re-types the oracle's loop):
* a hand-worked example (tests/golden/worked_example_d2_n3.txt);
* the quadratic closed form O = (Q K^T ⊙ M) V + Q S_0, S_N = S_0 + K^T V with the
  inclusive causal mask M (numpy matmul);
* exact integer brute force with Python ints over the double sum;
* special cases that reduce to cumsum / matmul;
* the chunked (block) evaluation at many block sizes, including non-divisors;
* continuation (split the sequence, carry the state) and linearity;
* the bf16 rounding against torch's conversion and the definition of RNE;
* planted mistakes in copies of the oracle that each pin must reject.
"""
import os

import numpy as np
import pytest

from oracle import oracle
from linear_attention_lightning_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, lead, N, d, with_state=True):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((*lead, N, d)) / np.sqrt(d)).astype(np.float32)
    k = (rng.standard_normal((*lead, N, d)) / np.sqrt(d)).astype(np.float32)
    v = rng.standard_normal((*lead, N, d)).astype(np.float32)
    S0 = rng.standard_normal((*lead, d, d)) if with_state else None
    return q, k, v, S0


def closed_form(q, k, v, S0):
    """(Q K^T ⊙ M) V + Q S_0 with M[r, c] = 1 iff c <= r, and S_0 + K^T V."""
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    N = q.shape[-2]
    M = np.tril(np.ones((N, N)))
    P = np.matmul(q64, np.swapaxes(k64, -1, -2)) * M
    O = np.matmul(P, v64)
    SN = np.matmul(np.swapaxes(k64, -1, -2), v64)
    if S0 is not None:
        O = O + np.matmul(q64, S0)
        SN = SN + S0
    return O, SN


def chunked_fp64(q, k, v, S0, blk):
    """Block evaluation written for the test: inside a block of ``blk`` tokens
    the masked product (Q_b K_b^T ⊙ M) V_b, plus Q_b S; then S += K_b^T V_b."""
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    *lead, N, d = q.shape
    S = np.zeros((*lead, d, d)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.empty((*lead, N, d))
    for s in range(0, N, blk):
        e = min(N, s + blk)
        Qb, Kb, Vb = q64[..., s:e, :], k64[..., s:e, :], v64[..., s:e, :]
        M = np.tril(np.ones((e - s, e - s)))
        O[..., s:e, :] = np.matmul(np.matmul(Qb, np.swapaxes(Kb, -1, -2)) * M, Vb) + np.matmul(Qb, S)
        S = S + np.matmul(np.swapaxes(Kb, -1, -2), Vb)
    return O, S


def rel_err(a, b):
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = [float(x) for x in rest.split()]
    d, N = int(vals["d"][0]), int(vals["N"][0])
    arr = {k: np.array(vals[k]) for k in ("q", "k", "v", "S0", "o", "SN")}
    return (arr["q"].reshape(N, d).astype(np.float32), arr["k"].reshape(N, d).astype(np.float32),
            arr["v"].reshape(N, d).astype(np.float32), arr["S0"].reshape(d, d),
            arr["o"].reshape(N, d), arr["SN"].reshape(d, d))


# ---------------------------------------------------------------- pins ----

def check_golden(rec):
    q, k, v, S0, o_ref, S_ref = load_golden("worked_example_d2_n3.txt")
    o, S = rec(q, k, v, S0)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(S, S_ref)


def check_closed_form(rec):
    for seed, lead, N, d in [(1, (1,), 1, 4), (2, (3,), 7, 16), (3, (2, 2), 64, 8), (4, (1,), 257, 64),
                             (5, (2,), 33, 5)]:
        q, k, v, S0 = rand_case(seed, lead, N, d)
        o, S = rec(q, k, v, S0)
        O_ref, S_ref = closed_form(q, k, v, S0)
        assert rel_err(o, O_ref) < 1e-12, (seed, rel_err(o, O_ref))
        assert rel_err(S, S_ref) < 1e-12, (seed, rel_err(S, S_ref))


def check_integer_bruteforce(rec):
    rng = np.random.default_rng(7)
    N, d = 9, 3
    q = rng.integers(-3, 4, size=(N, d))
    k = rng.integers(-3, 4, size=(N, d))
    v = rng.integers(-3, 4, size=(N, d))
    S0 = rng.integers(-3, 4, size=(d, d))
    # o_t[j] = sum_{s<=t} (sum_i q_t[i] k_s[i]) v_s[j] + sum_i q_t[i] S0[i][j], in Python ints
    o_ref = [[sum(sum(int(q[t, i]) * int(k[s, i]) for i in range(d)) * int(v[s, j]) for s in range(t + 1))
              + sum(int(q[t, i]) * int(S0[i, j]) for i in range(d)) for j in range(d)] for t in range(N)]
    S_ref = [[int(S0[i, j]) + sum(int(k[s, i]) * int(v[s, j]) for s in range(N)) for j in range(d)]
             for i in range(d)]
    o, S = rec(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), S0)
    np.testing.assert_array_equal(o, np.array(o_ref, dtype=np.float64))
    np.testing.assert_array_equal(S, np.array(S_ref, dtype=np.float64))


def check_cumsum_cases(rec):
    rng = np.random.default_rng(11)
    # d = 1: o_t = q_t * sum_{s<=t} k_s v_s (+ q_t S0)
    N = 50
    q, k, v = (rng.standard_normal((N, 1)).astype(np.float32) for _ in range(3))
    o, _ = rec(q, k, v, np.array([[0.25]]))
    ref = q[:, 0].astype(np.float64) * (np.cumsum(k[:, 0].astype(np.float64) * v[:, 0]) + 0.25)
    assert rel_err(o[:, 0], ref) < 1e-12
    # k_t = ones, q_t = e_i: o_t = sum_{s<=t} v_s (+ row i of S0)
    d, i = 6, 4
    v = rng.standard_normal((N, d)).astype(np.float32)
    k = np.ones((N, d), np.float32)
    q = np.zeros((N, d), np.float32)
    q[:, i] = 1
    S0 = rng.standard_normal((d, d))
    o, _ = rec(q, k, v, S0)
    assert rel_err(o, np.cumsum(v.astype(np.float64), axis=0) + S0[i]) < 1e-12
    # all v = 0 with S0: o = Q S0 (a plain matmul), state unchanged
    q = rng.standard_normal((N, d)).astype(np.float32)
    k = rng.standard_normal((N, d)).astype(np.float32)
    o, S = rec(q, k, np.zeros((N, d), np.float32), S0)
    assert rel_err(o, q.astype(np.float64) @ S0) < 1e-12
    np.testing.assert_array_equal(S, S0)


def check_chunked_equivalence(rec):
    q, k, v, S0 = rand_case(21, (2,), 100, 8)
    o, S = rec(q, k, v, S0)
    for blk in (1, 2, 3, 16, 64, 100, 128):
        Oc, Sc = chunked_fp64(q, k, v, S0, blk)
        assert rel_err(o, Oc) < 1e-12, blk
        assert rel_err(S, Sc) < 1e-12, blk


ALL_PINS = [check_golden, check_closed_form, check_integer_bruteforce, check_cumsum_cases,
            check_chunked_equivalence]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.recurrence)


def test_continuation_and_decode_steps():
    q, k, v, S0 = rand_case(31, (3,), 40, 8)
    o_all, S_all = oracle.recurrence(q, k, v, S0)
    for n in (0, 1, 17, 40):
        o1, S1 = oracle.recurrence(q[:, :n], k[:, :n], v[:, :n], S0)
        o2, S2 = oracle.recurrence(q[:, n:], k[:, n:], v[:, n:], S1)
        np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o_all)
        np.testing.assert_array_equal(S2, S_all)
    # token-at-a-time decode reproduces the sequence run bitwise
    S = np.array(S0, dtype=np.float64)
    for t in range(40):
        o_t = oracle.decode_step(q[:, t], k[:, t], v[:, t], S)
        np.testing.assert_array_equal(o_t, o_all[:, t])
    np.testing.assert_array_equal(S, S_all)


def test_linearity():
    q, k, _, S0 = rand_case(41, (2,), 30, 6)
    _, _, _, S02 = rand_case(42, (2,), 30, 6)
    # integer-valued v so that a*v + b*v2 is exact in float32
    rng = np.random.default_rng(44)
    v, v2 = (rng.integers(-8, 9, (2, 30, 6)).astype(np.float32) for _ in range(2))
    a, b = 0.75, -1.5
    o1, _ = oracle.recurrence(q, k, v, S0)
    o2, _ = oracle.recurrence(q, k, v2, S02)
    o12, _ = oracle.recurrence(q, k, (a * v + b * v2).astype(np.float32), a * S0 + b * S02)
    assert rel_err(o12, a * o1 + b * o2) < 1e-12
    # linear in q (integer-valued q's so that q + q2 is exact in float32)
    q = rng.integers(-4, 5, (2, 30, 6)).astype(np.float32)
    q2 = rng.integers(-4, 5, (2, 30, 6)).astype(np.float32)
    o1, _ = oracle.recurrence(q, k, v, S0)
    o_q2, _ = oracle.recurrence(q2, k, v, S0)
    o_sum, _ = oracle.recurrence((q + q2).astype(np.float32), k, v, S0)
    assert rel_err(o_sum, o1 + o_q2) < 1e-12


def test_state_after_is_the_recurrence_state():
    """The matrix-product form of the final state agrees with the token loop:
    exactly on integers, to fp64 rounding on random values, and it splits at
    any point (continuation)."""
    q, k, v = (x.astype(np.float32) for x in np.random.default_rng(41).integers(-3, 4, (3, 2, 3, 50, 8)))
    S0 = np.random.default_rng(42).integers(-5, 6, (2, 3, 8, 8)).astype(np.float64)
    _, S_ref = oracle.recurrence(q, k, v, S0)
    np.testing.assert_array_equal(oracle.state_after(k, v, S0), S_ref)
    q, k, v, S0 = rand_case(43, (2,), 300, 16)
    _, S_ref = oracle.recurrence(q, k, v, S0)
    S = oracle.state_after(k, v, S0)
    assert np.max(np.abs(S - S_ref)) <= 1e-12 * np.max(np.abs(S_ref))
    S_split = oracle.state_after(k[:, 120:], v[:, 120:], oracle.state_after(k[:, :120], v[:, :120], S0))
    assert np.max(np.abs(S_split - S_ref)) <= 1e-12 * np.max(np.abs(S_ref))
    assert np.array_equal(oracle.state_after(k[:, :0], v[:, :0], S0), S0)


def test_empty_inputs():
    q = np.zeros((2, 0, 4), np.float32)
    S0 = np.ones((2, 4, 4))
    o, S = oracle.recurrence(q, q, q, S0)
    assert o.shape == (2, 0, 4)
    np.testing.assert_array_equal(S, S0)


def test_oracle_error_bound_fp64():
    """Forward error of the fp64 recurrence is far below the GPU gates: a
    bf16-valued sequence of 4096 tokens computed in fp64 agrees with an exact
    rational-free re-evaluation (closed form) to ~1e-13."""
    q, k, v = synth.prefill_inputs(0, 1, 1, 4096, 16)
    o, S = oracle.recurrence(q, k, v)
    O_ref, S_ref = closed_form(q, k, v, None)
    assert rel_err(o, O_ref) < 1e-11
    assert rel_err(S, S_ref) < 1e-11


# ------------------------------------------------------ bf16 rounding ----

def test_round_bf16_matches_torch_on_float32_values():
    import torch
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-42], np.float32)]).astype(np.float32)
    # exact ties: bf16 grid points plus half a bf16 ulp
    base = torch.from_numpy(rng.standard_normal(4000).astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    bits = base.view(np.uint32) | np.uint32(0x8000)
    x = np.concatenate([x, bits.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16_bits(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_definition_on_doubles():
    """For doubles (not only float32 values): the result is a bf16 value,
    within half a bf16 ulp, and on exact ties its last fraction bit is 0."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)
    r = oracle.bf16_bits_to_f64(oracle.round_bf16_bits(x))
    e = np.floor(np.log2(np.abs(x)))
    ulp = 2.0 ** (e - 7)
    err = np.abs(x - r)
    assert np.all(err <= ulp / 2 * (1 + 1e-15))
    # construct exact ties in double: midpoint between two bf16 neighbours
    lo = oracle.bf16_bits_to_f64(np.arange(0x3f80, 0x3fff, dtype=np.uint16))
    hi = oracle.bf16_bits_to_f64(np.arange(0x3f81, 0x4000, dtype=np.uint16))
    mid = (lo + hi) / 2
    rb = oracle.round_bf16_bits(mid)
    assert np.all(rb % 2 == 0)


def test_decode_bf16_state_definition():
    rng = np.random.default_rng(8)
    d = 8
    q, k, v = (rng.standard_normal((3, d)).astype(np.float32) for _ in range(3))
    S = rng.standard_normal((3, d, d))
    Sb = oracle.round_bf16_bits(S)
    S_wide = oracle.bf16_bits_to_f64(Sb)
    o = oracle.decode_step_bf16_state(q, k, v, Sb)
    S_new = S_wide + k[:, :, None].astype(np.float64) * v[:, None, :]
    o_ref = np.einsum("hi,hij->hj", q.astype(np.float64), S_new)
    assert rel_err(o, o_ref) < 1e-14
    np.testing.assert_array_equal(Sb, oracle.round_bf16_bits(S_new))
    # exact-integer inputs: no rounding happens, so it equals the fp64 decode
    qi, ki, vi = (rng.integers(-2, 3, (4, d)).astype(np.float32) for _ in range(3))
    S0 = rng.integers(-5, 6, (4, d, d)).astype(np.float64)
    Sb = oracle.round_bf16_bits(S0)
    S64 = S0.copy()
    for _ in range(5):
        ob = oracle.decode_step_bf16_state(qi, ki, vi, Sb)
        o6 = oracle.decode_step(qi, ki, vi, S64)
        np.testing.assert_array_equal(ob, o6)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(Sb), S64)


# --------------------------------------------- planted mistakes (CPU) ----

MUTANTS = {
    # readout before the update: the exclusive mask
    "exclusive_mask": ("    /* S_t = S_{t-1} + k_t v_t^T */\n    for (int64_t i = 0; i < d; ++i) {\n      const double ki = (double)kt[i];\n      double *Si = S + i * d;\n      for (int64_t j = 0; j < d; ++j) Si[j] += ki * (double)vt[j];\n    }\n    /* o_t[j] = sum_i q_t[i] S_t[i][j] */\n    for (int64_t j = 0; j < d; ++j) ot[j] = 0.0;\n    for (int64_t i = 0; i < d; ++i) {\n      const double qi = (double)qt[i];\n      const double *Si = S + i * d;\n      for (int64_t j = 0; j < d; ++j) ot[j] += qi * Si[j];\n    }\n",
                       "    for (int64_t j = 0; j < d; ++j) ot[j] = 0.0;\n    for (int64_t i = 0; i < d; ++i) {\n      const double qi = (double)qt[i];\n      const double *Si = S + i * d;\n      for (int64_t j = 0; j < d; ++j) ot[j] += qi * Si[j];\n    }\n    for (int64_t i = 0; i < d; ++i) {\n      const double ki = (double)kt[i];\n      double *Si = S + i * d;\n      for (int64_t j = 0; j < d; ++j) Si[j] += ki * (double)vt[j];\n    }\n"),
    "sign_flip": ("Si[j] += ki * (double)vt[j];", "Si[j] -= ki * (double)vt[j];"),
    "transposed_state_read": ("for (int64_t j = 0; j < d; ++j) ot[j] += qi * Si[j];",
                              "for (int64_t j = 0; j < d; ++j) ot[j] += qi * S[j * d + i];"),
    "k_v_swapped": ("const double ki = (double)kt[i];", "const double ki = (double)vt[i];"),
    "dropped_query_weight": ("const double qi = (double)qt[i];", "const double qi = 1.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistakes(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation target for {name} not found verbatim in the oracle"
    variant = oracle.compile_variant(src.replace(old, new), str(tmp_path / f"mut_{name}.so"))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(variant.recurrence)
        except AssertionError:
            caught.append(pin.__name__)
    # every mutant must be rejected by the closed form and by the hand-worked example
    assert "check_closed_form" in caught, (name, caught)
    assert "check_golden" in caught or name == "dropped_query_weight" and "check_integer_bruteforce" in caught, (name, caught)
