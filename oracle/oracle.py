"""fp64 CPU oracle for causal linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library
(``linear_attention_lightning_amd``) and imports nothing from it.

The arithmetic lives in ``lin_attn_oracle.c`` (plain C, IEEE double, no
blocking or reordering): the token-by-token recurrence

    S_t = S_{t-1} + k_t v_t^T ,   o_t = q_t^T S_t

of "MiniMax-M1で理解する：大規模言語モデルのコンテキスト長限界を突破する革新的
アーキテクチャ" (zenn.dev/liushuzhi), section "線形アテンションの数学的基礎",
recurrence equations, with phi = identity.  This module only compiles that
file, marshals numpy arrays into it and back, and picks a thread count.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lin_attn_oracle.c")
_LIB = os.path.join(_HERE, "liblin_attn_oracle.so")

# Portable x86-64 target with AVX2 (runs on current Xeon and EPYC hosts);
# no -ffast-math, no FMA contraction, so every product and sum is
# a separately rounded IEEE double operation.
_CFLAGS = ["-O3", "-std=c11", "-march=x86-64-v3", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-pthread"]

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library in place and return its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.lao_recurrence.argtypes = [p, p, p, p, p, i64, i64, i64, ctypes.c_int]
    lib.lao_recurrence.restype = ctypes.c_int
    lib.lao_decode_bf16_state.argtypes = [p, p, p, p, p, i64, i64, ctypes.c_int]
    lib.lao_decode_bf16_state.restype = ctypes.c_int
    lib.lao_round_bf16.argtypes = [p, p, i64]
    lib.lao_round_bf16.restype = None
    lib.lao_recurrence_stored_state.argtypes = [p, p, p, p, p, ctypes.c_int, p, i64, i64, i64, i64,
                                                ctypes.c_int]
    lib.lao_recurrence_stored_state.restype = ctypes.c_int
    lib.lao_round_e4m3.argtypes = [p, p, i64]
    lib.lao_round_e4m3.restype = None
    lib.lao_widen_e4m3.argtypes = [p, p, i64]
    lib.lao_widen_e4m3.restype = None
    lib.lao_backward.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i64, i64, ctypes.c_int]
    lib.lao_backward.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = _bind(_LIB)
    return _lib


def compile_variant(src_text: str, out_path: str):
    """Compile C source text with the oracle's flags and bind it like the
    oracle.  Used by the tests to plant a mistake in a copy of the oracle and
    show that the pins catch it; returns an object whose ``recurrence``
    behaves like :func:`recurrence`."""
    src_path = out_path + ".c"
    with open(src_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *_CFLAGS, "-o", out_path, src_path, "-lm"], check=True)
    lib = _bind(out_path)

    class _Variant:
        @staticmethod
        def recurrence(q, k, v, S0=None, nthreads=None):
            return recurrence(q, k, v, S0, nthreads, _lib_obj=lib)

        @staticmethod
        def round_e4m3_codes(x):
            return round_e4m3_codes(x, _lib_obj=lib)

        @staticmethod
        def e4m3_codes_to_f64(codes):
            return e4m3_codes_to_f64(codes, _lib_obj=lib)

        @staticmethod
        def round_to_stored(x, fmt, scale=None):
            return round_to_stored(x, fmt, scale, _lib_obj=lib)

        @staticmethod
        def stored_to_f64(codes, fmt, scale=None):
            return stored_to_f64(codes, fmt, scale, _lib_obj=lib)

        @staticmethod
        def backward(q, k, v, dout, S0=None, dSN=None, nthreads=None):
            return backward(q, k, v, dout, S0, dSN, nthreads, _lib_obj=lib)

        @staticmethod
        def recurrence_stored_state(q, k, v, codes, fmt, scale=None, block=1, nthreads=None):
            return recurrence_stored_state(q, k, v, codes, fmt, scale, block, nthreads, _lib_obj=lib)

    return _Variant()


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def default_threads() -> int:
    """Host threads to use: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when that is set (it bounds the process's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _f32(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32)
    if a.dtype != np.float32:
        raise TypeError("expected float32-convertible input")
    return a


def recurrence(q, k, v, S0=None, nthreads: int | None = None, _lib_obj=None):
    """Causal linear attention by the token-by-token fp64 recurrence.

    q, k, v: arrays of shape [..., N, d] holding fp32 (or bf16-valued fp32)
    numbers; the leading axes enumerate independent (batch, head) pairs.
    S0: optional [..., d, d] initial state (zeros when omitted).
    Returns (o, S_N): o float64 [..., N, d] and S_N float64 [..., d, d].
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    if not (q.shape == k.shape == v.shape) or q.ndim < 2:
        raise ValueError(f"q, k, v must share a shape [..., N, d]; got {q.shape}, {k.shape}, {v.shape}")
    *lead, N, d = q.shape
    nheads = int(np.prod(lead)) if lead else 1
    if S0 is None:
        S = np.zeros((*lead, d, d), dtype=np.float64)
    else:
        S = np.array(S0, dtype=np.float64, order="C", copy=True)
        if S.shape != (*lead, d, d):
            raise ValueError(f"S0 must have shape {(*lead, d, d)}; got {S.shape}")
    o = np.empty((*lead, N, d), dtype=np.float64)
    if nheads == 0 or N == 0:
        return o, S
    lib = _lib_obj if _lib_obj is not None else _load()
    rc = lib.lao_recurrence(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                            S.ctypes.data, nheads, N, d, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle recurrence failed with code {rc}")
    return o, S


def decode_step(q, k, v, S, nthreads: int | None = None):
    """One decode token per head: S <- S + k v^T ; o = q^T S (fp64, in place
    on the float64 array ``S``).  q, k, v: [..., d]; S: [..., d, d] float64.
    Returns o float64 [..., d]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    if not isinstance(S, np.ndarray) or S.dtype != np.float64 or not S.flags.c_contiguous:
        raise TypeError("S must be a C-contiguous float64 array (updated in place)")
    *lead, d = q.shape
    if S.shape != (*lead, d, d):
        raise ValueError(f"S must have shape {(*lead, d, d)}; got {S.shape}")
    nheads = int(np.prod(lead)) if lead else 1
    o = np.empty((*lead, d), dtype=np.float64)
    if nheads == 0:
        return o
    rc = _load().lao_recurrence(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                                S.ctypes.data, nheads, 1, d, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle decode failed with code {rc}")
    return o


def decode_step_bf16_state(q, k, v, S_bits, nthreads: int | None = None):
    """One decode token per head with the state kept in bf16 between steps.

    S_bits: uint16 array [..., d, d] of bf16 bit patterns, updated in place:
    widened to double, S += k v^T, o = q^T S read from the double value, then
    stored back rounded to nearest-even bf16.  Returns o float64 [..., d]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    if not isinstance(S_bits, np.ndarray) or S_bits.dtype != np.uint16 or not S_bits.flags.c_contiguous:
        raise TypeError("S_bits must be a C-contiguous uint16 array (updated in place)")
    *lead, d = q.shape
    if S_bits.shape != (*lead, d, d):
        raise ValueError(f"S_bits must have shape {(*lead, d, d)}; got {S_bits.shape}")
    nheads = int(np.prod(lead)) if lead else 1
    o = np.empty((*lead, d), dtype=np.float64)
    if nheads == 0:
        return o
    rc = _load().lao_decode_bf16_state(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                                       S_bits.ctypes.data, nheads, d, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle bf16-state decode failed with code {rc}")
    return o


def round_bf16_bits(x, _lib_obj=None) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); uint16 bit patterns."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    (_lib_obj or _load()).lao_round_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64 (a bit shift)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


FMT_BF16 = 1
FMT_E4M3 = 2
_CODE_DTYPE = {FMT_BF16: np.uint16, FMT_E4M3: np.uint8}


def round_e4m3_codes(x, _lib_obj=None) -> np.ndarray:
    """Round float64 values to OCP FP8 E4M3 (nearest, ties to even, clamped to
    +-448; NaN stays NaN); uint8 codes."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint8)
    (_lib_obj or _load()).lao_round_e4m3(a.ctypes.data, out.ctypes.data, a.size)
    return out


def e4m3_codes_to_f64(codes, _lib_obj=None) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 codes as float64 (NaN for S.1111.111)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    (_lib_obj or _load()).lao_widen_e4m3(c.ctypes.data, out.ctypes.data, c.size)
    return out


def stored_to_f64(codes, fmt: int, scale=None, _lib_obj=None) -> np.ndarray:
    """Value of a stored state: value(code) * scale, scale per head ([...]) or None."""
    val = bf16_bits_to_f64(codes) if fmt == FMT_BF16 else e4m3_codes_to_f64(codes, _lib_obj)
    if scale is not None:
        val = val * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None, None]
    return val


def round_to_stored(x, fmt: int, scale=None, _lib_obj=None) -> np.ndarray:
    """Codes of x / scale in the stored format."""
    x = np.asarray(x, dtype=np.float64)
    if scale is not None:
        x = x / np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None, None]
    return round_bf16_bits(x, _lib_obj) if fmt == FMT_BF16 else round_e4m3_codes(x, _lib_obj)


def recurrence_stored_state(q, k, v, codes, fmt: int, scale=None, block: int = 1,
                            nthreads: int | None = None, _lib_obj=None):
    """Recurrence whose state is stored in a narrow format every `block`
    tokens and after the last one.

    codes: C-contiguous [..., d, d] uint16 (fmt FMT_BF16) or uint8 (FMT_E4M3)
    array, updated in place (in: S_0, out: S_N); scale: float32 [...] per
    head or None for 1.  Returns o float64 [..., N, d]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    if fmt not in _CODE_DTYPE:
        raise ValueError("fmt must be FMT_BF16 or FMT_E4M3")
    if not isinstance(codes, np.ndarray) or codes.dtype != _CODE_DTYPE[fmt] or not codes.flags.c_contiguous:
        raise TypeError(f"codes must be a C-contiguous {np.dtype(_CODE_DTYPE[fmt]).name} array (updated in place)")
    *lead, N, d = q.shape
    if codes.shape != (*lead, d, d):
        raise ValueError(f"codes must have shape {(*lead, d, d)}; got {codes.shape}")
    nheads = int(np.prod(lead)) if lead else 1
    sc = None
    if scale is not None:
        sc = np.ascontiguousarray(np.broadcast_to(np.asarray(scale, dtype=np.float32), tuple(lead)))
    o = np.empty((*lead, N, d), dtype=np.float64)
    if nheads == 0 or N == 0:
        return o
    rc = (_lib_obj or _load()).lao_recurrence_stored_state(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                                             codes.ctypes.data, fmt, None if sc is None else sc.ctypes.data,
                                             nheads, N, d, block, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle stored-state recurrence failed with code {rc}")
    return o


def state_after(k, v, S0=None) -> np.ndarray:
    """The recurrence's state after the tokens of k, v: S_N = S_0 + sum_t
    k_t v_t^T, in float64, as one matrix product K^T V per head (the sum the
    recurrence accumulates, without the outputs; for long sequences whose
    outputs are not needed).  k, v: [..., N, d]; S0: [..., d, d] or None."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S = np.matmul(np.swapaxes(k, -1, -2), v)
    if S0 is not None:
        S = S + np.asarray(S0, dtype=np.float64)
    return S


def backward(q, k, v, dout, S0=None, dSN=None, nthreads: int | None = None, _lib_obj=None):
    """Gradients of L = sum_t <o_t, dout_t> + <S_N, dSN> through the
    recurrence: returns (dq, dk, dv, dS0) as float64 arrays.

    q, k, v, dout: [..., N, d] (fp32 or bf16-valued fp32); S0, dSN:
    [..., d, d] or None (zero)."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    *lead, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have shape {q.shape}; got {t.shape}")

    def st(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x, dtype=np.float64)
        if x.shape != (*lead, d, d):
            raise ValueError(f"states must have shape {(*lead, d, d)}; got {x.shape}")
        return x

    S0, dSN = st(S0), st(dSN)
    nheads = int(np.prod(lead)) if lead else 1
    dq = np.empty((*lead, N, d))
    dk = np.empty((*lead, N, d))
    dv = np.empty((*lead, N, d))
    dS0 = np.empty((*lead, d, d))
    if nheads == 0:
        return dq, dk, dv, dS0
    rc = (_lib_obj or _load()).lao_backward(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                            None if S0 is None else S0.ctypes.data,
                                            None if dSN is None else dSN.ctypes.data,
                                            dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, dS0.ctypes.data,
                                            nheads, N, d, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle backward failed with code {rc}")
    return dq, dk, dv, dS0
