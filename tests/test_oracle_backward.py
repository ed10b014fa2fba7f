"""Pins of the oracle's gradients (the backward pass of the recurrence)
against facts that do not come from the oracle.

What is pinned: for L = sum_t <o_t, dO_t> + <S_N, dS_N> with the recurrence
S_t = S_{t-1} + k_t v_t^T, o_t = q_t^T S_t ("MiniMax-M1で理解する…"
(zenn.dev/liushuzhi), section "線形アテンションの数学的基礎"), the oracle
returns dq, dk, dv and dS_0 from a forward loop (dq_t = S_t dO_t) and a loop
that carries G_t = dS_N + sum_{r >= t} q_r dO_r^T backwards.

Pins used:
* finite differences of the forward oracle: L is linear in each of q, k, v
  and S_0 taken alone, so a central difference along any direction equals
  the directional derivative exactly (inputs and steps on a grid that
  float32 holds exactly);
* the closed-form gradient of O = (Q K^T ⊙ M) V + Q S_0, S_N = S_0 + K^T V,
  written with numpy matrix products (exact on integers);
* special cases: N = 0 and N = 1;
* planted mistakes in copies of the oracle that the pins must reject.
"""
import numpy as np
import pytest

from oracle import oracle


def grid_case(seed, lead, N, d):
    """Inputs on the grid of multiples of 1/8 in [-2, 2] (exact in float32)."""
    rng = np.random.default_rng(seed)
    q, k, v, dO = (rng.integers(-16, 17, (*lead, N, d)).astype(np.float32) / 8 for _ in range(4))
    S0 = rng.integers(-16, 17, (*lead, d, d)) / 8.0
    dSN = rng.integers(-16, 17, (*lead, d, d)) / 8.0
    return q, k, v, dO, S0, dSN


def loss(q, k, v, dO, S0, dSN):
    o, S = oracle.recurrence(q, k, v, S0)
    return float(np.sum(o * dO) + np.sum(S * dSN))


def check_finite_differences(lib=oracle):
    q, k, v, dO, S0, dSN = grid_case(51, (2,), 9, 4)
    dq, dk, dv, dS0 = lib.backward(q, k, v, dO, S0, dSN)
    rng = np.random.default_rng(52)
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("S0", dS0)):
        for _ in range(3):
            u = rng.integers(-2, 3, grad.shape) / 4.0  # on the 1/8 grid after the 0.5 step
            args = {"q": q, "k": k, "v": v, "S0": S0}

            def at(sign):
                a = dict(args)
                x = a[name] + sign * 0.5 * u
                a[name] = x.astype(np.float32) if name != "S0" else x
                return loss(a["q"], a["k"], a["v"], dO, a["S0"], dSN)

            fd = (at(+1) - at(-1)) / 1.0  # (L(x + u/2) - L(x - u/2)) / (2 * 0.5)
            dd = float(np.sum(grad * u))
            assert abs(fd - dd) <= 1e-12 * max(1.0, abs(dd)), (name, fd, dd)


def closed_form(q, k, v, dO, S0, dSN):
    q, k, v, dO = (np.asarray(x, np.float64) for x in (q, k, v, dO))
    N = q.shape[-2]
    M = np.tril(np.ones((N, N)))
    kT = np.swapaxes(k, -1, -2)
    qT = np.swapaxes(q, -1, -2)
    vT = np.swapaxes(v, -1, -2)
    dOT = np.swapaxes(dO, -1, -2)
    dq = ((dO @ vT) * M) @ k + dO @ np.swapaxes(S0, -1, -2)
    dk = ((v @ dOT) * M.T) @ q + v @ np.swapaxes(dSN, -1, -2)
    dv = ((k @ qT) * M.T) @ dO + k @ dSN
    dS0 = qT @ dO + dSN
    return dq, dk, dv, dS0


def check_closed_form(lib=oracle):
    # exact on integers
    rng = np.random.default_rng(53)
    q, k, v, dO = (rng.integers(-3, 4, (2, 3, 20, 5)).astype(np.float32) for _ in range(4))
    S0, dSN = (rng.integers(-3, 4, (2, 3, 5, 5)).astype(np.float64) for _ in range(2))
    for got, ref in zip(lib.backward(q, k, v, dO, S0, dSN), closed_form(q, k, v, dO, S0, dSN)):
        np.testing.assert_array_equal(got, ref)
    # random reals, 300 tokens
    q, k, v, dO = (rng.standard_normal((2, 300, 16)).astype(np.float32) for _ in range(4))
    S0, dSN = (rng.standard_normal((2, 16, 16)) for _ in range(2))
    for got, ref in zip(lib.backward(q, k, v, dO, S0, dSN), closed_form(q, k, v, dO, S0, dSN)):
        assert np.max(np.abs(got - ref)) <= 1e-11 * np.max(np.abs(ref))


def check_special_cases(lib=oracle):
    rng = np.random.default_rng(54)
    d = 6
    S0, dSN = rng.standard_normal((2, d, d)), rng.standard_normal((2, d, d))
    e = np.zeros((2, 0, d), np.float32)
    dq, dk, dv, dS0 = lib.backward(e, e, e, e, S0, dSN)
    assert dq.shape == (2, 0, d) and np.array_equal(dS0, dSN)
    q, k, v, dO = (rng.standard_normal((2, 1, d)).astype(np.float32) for _ in range(4))
    dq, dk, dv, dS0 = lib.backward(q, k, v, dO, S0, dSN)
    q64, k64, v64, dO64 = (x[:, 0].astype(np.float64) for x in (q, k, v, dO))
    S1 = S0 + k64[:, :, None] * v64[:, None, :]
    G = dSN + q64[:, :, None] * dO64[:, None, :]
    assert np.allclose(dq[:, 0], np.einsum("hij,hj->hi", S1, dO64), rtol=0, atol=1e-12)
    assert np.allclose(dk[:, 0], np.einsum("hij,hj->hi", G, v64), rtol=0, atol=1e-12)
    assert np.allclose(dv[:, 0], np.einsum("hij,hi->hj", G, k64), rtol=0, atol=1e-12)
    assert np.allclose(dS0, G, rtol=0, atol=1e-12)
    # no final-state gradient and no initial state: None means zero
    a = lib.backward(q, k, v, dO, None, None)
    b = lib.backward(q, k, v, dO, np.zeros_like(S0), np.zeros_like(dSN))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


BWD_PINS = [check_finite_differences, check_closed_form, check_special_cases]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin()


BWD_MUTANTS = {
    # G updated after the token's own dk, dv (the exclusive reverse sum)
    "exclusive_reverse_carry": (
        "    for (int64_t i = 0; i < d; ++i) {\n      const double qri = (double)qt[i];\n      for (int64_t j = 0; j < d; ++j) G[i * d + j] += qri * (double)dot[j];\n    }\n    for (int64_t i = 0; i < d; ++i) {\n      double acc = 0.0;\n      for (int64_t j = 0; j < d; ++j) acc += G[i * d + j] * (double)vt[j];\n      dk[t * d + i] = acc;\n    }\n",
        "    for (int64_t i = 0; i < d; ++i) {\n      double acc = 0.0;\n      for (int64_t j = 0; j < d; ++j) acc += G[i * d + j] * (double)vt[j];\n      dk[t * d + i] = acc;\n    }\n    for (int64_t i = 0; i < d; ++i) {\n      const double qri = (double)qt[i];\n      for (int64_t j = 0; j < d; ++j) G[i * d + j] += qri * (double)dot[j];\n    }\n"),
    "dk_with_transposed_carry": ("for (int64_t j = 0; j < d; ++j) acc += G[i * d + j] * (double)vt[j];",
                                 "for (int64_t j = 0; j < d; ++j) acc += G[j * d + i] * (double)vt[j];"),
    "dq_from_transposed_state": ("for (int64_t j = 0; j < d; ++j) acc += S[i * d + j] * (double)dot[j];",
                                 "for (int64_t j = 0; j < d; ++j) acc += S[j * d + i] * (double)dot[j];"),
    "dv_weights_from_v": ("const double kbi = (double)kt[i];\n      for (int64_t j = 0; j < d; ++j) dv[t * d + j] += G[i * d + j] * kbi;",
                          "const double kbi = (double)vt[i];\n      for (int64_t j = 0; j < d; ++j) dv[t * d + j] += G[i * d + j] * kbi;"),
    "final_state_gradient_dropped": ("for (int64_t i = 0; i < d * d; ++i) G[i] = dSN ? dSN[i] : 0.0;",
                                     "for (int64_t i = 0; i < d * d; ++i) G[i] = 0.0;"),
    "initial_state_dropped": ("for (int64_t i = 0; i < dd; ++i) S[i] = jb->S0 ? jb->S0[h * dd + i] : 0.0;",
                              "for (int64_t i = 0; i < dd; ++i) S[i] = 0.0;"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_pins_reject_planted_mistakes(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation target for {name} not found verbatim in the oracle"
    variant = oracle.compile_variant(src.replace(old, new), str(tmp_path / f"mut_{name}.so"))
    caught = []
    for pin in BWD_PINS:
        try:
            pin(variant)
        except AssertionError:
            caught.append(pin.__name__)
    assert "check_finite_differences" in caught, (name, caught)
    assert "check_closed_form" in caught, (name, caught)
