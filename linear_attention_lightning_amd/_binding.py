"""ctypes binding of the C ABI in include/lin_attn.h.

Argument marshalling only: shape/dtype/device checks, pointer extraction and
the current HIP stream.  Every step of the computation runs in the gfx950
kernels of ``_lib/liblin_attn.so``; there is no other implementation here,
and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "liblin_attn.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
OK, EINVAL, EUNSUPPORTED, EHIP, ESCRATCH = 0, -1, -2, -3, -4

_lock = threading.Lock()
_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where} failed: {strerror(code)} (code {code})")


def library() -> ctypes.CDLL:
    """Load the HIP library (built by ``python -m linear_attention_lightning_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library not found at {LIB_PATH}; build it with "
                    "`python -m linear_attention_lightning_amd.build` (hipcc, gfx950)")
            lib = ctypes.CDLL(LIB_PATH)
            p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            lib.lin_attn_prefill.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32, p]
            lib.lin_attn_prefill.restype = i32
            lib.lin_attn_prefill_ex.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32, i64, p]
            lib.lin_attn_prefill_ex.restype = i32
            lib.lin_attn_decode.argtypes = [p, p, p, p, p, i64, i64, i64, i32, i32, p]
            lib.lin_attn_decode.restype = i32
            lib.lin_attn_decode_scaled.argtypes = [p, p, p, p, p, p, i64, i64, i64, i32, i32, p]
            lib.lin_attn_decode_scaled.restype = i32
            lib.lin_attn_prefill_scaled.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i32, i32, i64, p]
            lib.lin_attn_prefill_scaled.restype = i32
            lib.lin_attn_prefill_recurrent.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, p]
            lib.lin_attn_prefill_recurrent.restype = i32
            lib.lin_attn_prefill_snapshots.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32, p]
            lib.lin_attn_prefill_snapshots.restype = i32
            lib.lin_attn_decode_verify.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, i32, p]
            lib.lin_attn_decode_verify.restype = i32
            lib.lin_attn_decode_commit.argtypes = [p, p, p, p, i64, i64, i64, i64, i32, i32, p]
            lib.lin_attn_decode_commit.restype = i32
            lib.lin_attn_state_accumulate.argtypes = [p, p, p, i64, i64, i64, i64, i32, p]
            lib.lin_attn_state_accumulate.restype = i32
            lib.lin_attn_state_accumulate_split_workspace.argtypes = [i64, i64, i64, i64, i32]
            lib.lin_attn_state_accumulate_split_workspace.restype = i64
            lib.lin_attn_state_accumulate_split.argtypes = [p, p, p, i64, i64, i64, i64, i32, p, i64, p]
            lib.lin_attn_state_accumulate_split.restype = i32
            lib.lin_attn_prefill_seqsplit_workspace.argtypes = [i64, i64, i64, i64, i64, i32]
            lib.lin_attn_prefill_seqsplit_workspace.restype = i64
            lib.lin_attn_prefill_seqsplit.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32, p, i64, p]
            lib.lin_attn_prefill_seqsplit.restype = i32
            lib.lin_attn_scratch_bytes.argtypes = []
            lib.lin_attn_scratch_bytes.restype = i64
            lib.lin_attn_prefill_seqsplit_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32, p]
            lib.lin_attn_prefill_seqsplit_noalloc.restype = i32
            lib.lin_attn_decode_verify_scaled.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, p]
            lib.lin_attn_decode_verify_scaled.restype = i32
            lib.lin_attn_decode_commit_scaled.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, i32, p]
            lib.lin_attn_decode_commit_scaled.restype = i32
            lib.lin_attn_backward.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i32, p]
            lib.lin_attn_backward.restype = i32
            lib.lin_attn_backward_ex.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i32, i64, p]
            lib.lin_attn_backward_ex.restype = i32
            lib.lin_attn_strerror.argtypes = [i32]
            lib.lin_attn_strerror.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def strerror(code: int) -> str:
    return library().lin_attn_strerror(int(code)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}; expected torch.bfloat16, torch.float32 "
                    "(or torch.float8_e4m3fn for a stored state)")


def _scale_ptr(scale, B: int, H: int, device):
    """Device pointer of a float32 [B, H] scale tensor, or None."""
    import torch
    if scale is None:
        return None
    _check(scale, "state_scale", (B, H), torch.float32, device)
    return scale.data_ptr()


def _check(t, name: str, shape, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def prefill(q, k, v, o, state, block: int, *, split: int = 0, stream=None):
    """Chunked causal linear-attention prefill (``lin_attn_prefill_ex``).

    q, k, v, o: [B, H, N, d] bf16 or fp32 (one dtype for all four), contiguous,
    on one HIP device; state: [B, H, d, d] fp32, S_0 on entry, S_N on return
    (in place).  ``split`` = value-column slices per sequence (0 = automatic).
    Enqueued on ``stream`` (default: the current torch stream)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, (B, H, N, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), torch.float32, q.device)
    rc = library().lin_attn_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       state.data_ptr(), B, H, N, d, int(block), _dtype_code(q),
                                       int(split), _stream(stream, q.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_prefill")
    return o


def decode(q, k, v, o, state, *, state_scale=None, stream=None):
    """One decode token per sequence (``lin_attn_decode``, or
    ``lin_attn_decode_scaled`` when ``state_scale`` is given).

    q, k, v, o: [B, H, d] bf16 or fp32; state: [B, H, d, d] fp32, bf16 or
    float8_e4m3fn, updated in place; state_scale: optional float32 [B, H] on
    the device (narrow states: entry x is stored as x / scale)."""
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d]")
    B, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, (B, H, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), None, q.device)
    if state_scale is None:
        rc = library().lin_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       state.data_ptr(), B, H, d, _dtype_code(q), _dtype_code(state),
                                       _stream(stream, q.device))
        where = "lin_attn_decode"
    else:
        rc = library().lin_attn_decode_scaled(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                              state.data_ptr(), _scale_ptr(state_scale, B, H, q.device),
                                              B, H, d, _dtype_code(q), _dtype_code(state),
                                              _stream(stream, q.device))
        where = "lin_attn_decode_scaled"
    if rc != OK:
        raise LinAttnError(rc, where)
    return o


def prefill_scaled(q, k, v, o, state, block: int, *, state_scale=None, round_carry: bool = False,
                   stream=None):
    """Chunked prefill with the state stored as bf16 or float8_e4m3fn codes
    of state / scale (``lin_attn_prefill_scaled``).

    q, k, v, o: [B, H, N, d] bf16; state: [B, H, d, d] bf16 or
    float8_e4m3fn, S_0 on entry, S_N on return; state_scale: optional
    float32 [B, H] on the device; round_carry: round the carry to the
    state's format after every block."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, (B, H, N, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), None, q.device)
    if state.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError("state must be bfloat16 or float8_e4m3fn (use prefill for an fp32 state)")
    rc = library().lin_attn_prefill_scaled(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                           state.data_ptr(), _scale_ptr(state_scale, B, H, q.device),
                                           B, H, N, d, int(block), _dtype_code(q), _dtype_code(state),
                                           1 if round_carry else 0, _stream(stream, q.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_prefill_scaled")
    return o


def prefill_recurrent(q, k, v, o, state, *, stream=None):
    """Token-by-token prefill (``lin_attn_prefill_recurrent``); same tensors
    as :func:`prefill` without the block size."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, (B, H, N, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), torch.float32, q.device)
    rc = library().lin_attn_prefill_recurrent(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                              state.data_ptr(), B, H, N, d, _dtype_code(q),
                                              _stream(stream, q.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_prefill_recurrent")
    return o


def state_accumulate(k, v, state, *, stream=None):
    """state += K^T V over the N tokens of k, v (``lin_attn_state_accumulate``).

    k, v: [B, H, N, d] bf16 or fp32 (same dtype); state: [B, H, d, d] fp32,
    updated in place."""
    import torch
    if k.dim() != 4:
        raise ValueError("k must be [B, H, N, d]")
    B, H, N, d = k.shape
    _check(v, "v", (B, H, N, d), k.dtype, k.device)
    _check(k, "k", (B, H, N, d), k.dtype, k.device)
    _check(state, "state", (B, H, d, d), torch.float32, k.device)
    rc = library().lin_attn_state_accumulate(k.data_ptr(), v.data_ptr(), state.data_ptr(), B, H, N, d,
                                             _dtype_code(k), _stream(stream, k.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_state_accumulate")
    return state


def state_accumulate_split_workspace(B: int, H: int, N: int, d: int, dtype) -> int:
    """Workspace bytes ``state_accumulate_split`` needs for these sizes and
    the torch dtype of k and v (``lin_attn_state_accumulate_split_workspace``)."""
    import torch
    code = {torch.float32: F32, torch.bfloat16: BF16}.get(dtype)
    if code is None:
        raise LinAttnError(EUNSUPPORTED, "lin_attn_state_accumulate_split_workspace")
    n = library().lin_attn_state_accumulate_split_workspace(B, H, N, d, code)
    if n < 0:
        raise LinAttnError(int(n), "lin_attn_state_accumulate_split_workspace")
    return int(n)


def state_accumulate_split(k, v, state, workspace=None, *, stream=None):
    """state += K^T V with the tokens cut into chunks, one workgroup per
    (sequence, chunk), chunk sums added in chunk order
    (``lin_attn_state_accumulate_split``).

    k, v: [B, H, N, d] bf16 or fp32 (same dtype); state: [B, H, d, d] fp32,
    updated in place; workspace: a uint8 device tensor of at least
    ``state_accumulate_split_workspace(...)`` bytes, or None to allocate one
    here."""
    import torch
    if k.dim() != 4:
        raise ValueError("k must be [B, H, N, d]")
    B, H, N, d = k.shape
    _check(v, "v", (B, H, N, d), k.dtype, k.device)
    _check(k, "k", (B, H, N, d), k.dtype, k.device)
    _check(state, "state", (B, H, d, d), torch.float32, k.device)
    need = state_accumulate_split_workspace(B, H, N, d, k.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=k.device)
    if workspace.dtype != torch.uint8 or workspace.device != k.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the device of k")
    rc = library().lin_attn_state_accumulate_split(k.data_ptr(), v.data_ptr(), state.data_ptr(), B, H, N, d,
                                                   _dtype_code(k), workspace.data_ptr(), workspace.numel(),
                                                   _stream(stream, k.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_state_accumulate_split")
    return state


def prefill_seqsplit_workspace(B: int, H: int, N: int, d: int, block: int, dtype) -> int:
    """Workspace bytes ``prefill_seqsplit`` needs (``lin_attn_prefill_seqsplit_workspace``)."""
    import torch
    code = {torch.float32: F32, torch.bfloat16: BF16}.get(dtype)
    if code is None:
        raise LinAttnError(EUNSUPPORTED, "lin_attn_prefill_seqsplit_workspace")
    n = library().lin_attn_prefill_seqsplit_workspace(B, H, N, d, int(block), code)
    if n < 0:
        raise LinAttnError(int(n), "lin_attn_prefill_seqsplit_workspace")
    return int(n)


def prefill_seqsplit(q, k, v, o, state, block: int = 128, workspace=None, *, stream=None):
    """Chunked prefill with each sequence cut into parts along the tokens
    (``lin_attn_prefill_seqsplit``): the parts' initial states come from the
    K^T V of the parts before them, and the parts run as independent
    sequences.  Same arguments as ``prefill``; workspace: a uint8 device
    tensor of at least ``prefill_seqsplit_workspace(...)`` bytes, or None to
    allocate one here."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, n, (B, H, N, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), torch.float32, q.device)
    need = prefill_seqsplit_workspace(B, H, N, d, block, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the device of q")
    rc = library().lin_attn_prefill_seqsplit(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                             state.data_ptr(), B, H, N, d, int(block), _dtype_code(q),
                                             workspace.data_ptr(), workspace.numel(), _stream(stream, q.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_prefill_seqsplit")
    return o


def scratch_bytes() -> int:
    """Size of the library's fixed per-device scratch buffer (``lin_attn_scratch_bytes``)."""
    return int(library().lin_attn_scratch_bytes())


def prefill_seqsplit_noalloc(q, k, v, o, state, block: int = 128, *, stream=None):
    """``prefill_seqsplit`` with the workspace taken from the library's fixed
    per-device scratch buffer (``lin_attn_prefill_seqsplit_noalloc``): no
    device memory is allocated, here or in the library.  Calls that overlap
    on one device race on that buffer."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, n, (B, H, N, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), torch.float32, q.device)
    rc = library().lin_attn_prefill_seqsplit_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                     state.data_ptr(), B, H, N, d, int(block), _dtype_code(q),
                                                     _stream(stream, q.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_prefill_seqsplit_noalloc")
    return o


def snapshot_count(N: int, block: int, every: int) -> int:
    """Number of state snapshots lin_attn_prefill_snapshots writes per sequence."""
    return (N // block) // every


def prefill_snapshots(q, k, v, o, state, snapshots, block: int, every: int, *, stream=None):
    """:func:`prefill` that also writes state snapshots
    (``lin_attn_prefill_snapshots``): snapshots[b, h, s] = the state after
    (s + 1) * every * block tokens; snapshots is [B, H, nsnap, d, d] fp32 with
    nsnap = snapshot_count(N, block, every)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, (B, H, N, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), torch.float32, q.device)
    if every < 1:
        raise ValueError("every must be >= 1")
    nsnap = snapshot_count(N, block, every)
    _check(snapshots, "snapshots", (B, H, nsnap, d, d), torch.float32, q.device)
    rc = library().lin_attn_prefill_snapshots(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                              state.data_ptr(), snapshots.data_ptr() if nsnap else None,
                                              B, H, N, d, int(block), int(every), _dtype_code(q),
                                              _stream(stream, q.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_prefill_snapshots")
    return o


def decode_verify(q, k, v, o, state, *, state_scale=None, stream=None):
    """Outputs of T draft tokens per sequence from one read of the state
    (``lin_attn_decode_verify``, or ``lin_attn_decode_verify_scaled`` when
    ``state_scale`` is given); the state is not modified.

    q, k, v, o: [B, H, T, d] bf16 or fp32; state: [B, H, d, d] fp32, bf16 or
    float8_e4m3fn; state_scale: optional float32 [B, H] on the device."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, (B, H, T, d), q.dtype, q.device)
    _check(state, "state", (B, H, d, d), None, q.device)
    if state_scale is None:
        rc = library().lin_attn_decode_verify(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                              state.data_ptr(), B, H, T, d, _dtype_code(q), _dtype_code(state),
                                              _stream(stream, q.device))
        where = "lin_attn_decode_verify"
    else:
        rc = library().lin_attn_decode_verify_scaled(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                     state.data_ptr(), _scale_ptr(state_scale, B, H, q.device),
                                                     B, H, T, d, _dtype_code(q), _dtype_code(state),
                                                     _stream(stream, q.device))
        where = "lin_attn_decode_verify_scaled"
    if rc != OK:
        raise LinAttnError(rc, where)
    return o


def decode_commit(k, v, state, accept=None, *, state_scale=None, stream=None):
    """state += sum over the first accept[b] drafts of k v^T
    (``lin_attn_decode_commit``, or ``lin_attn_decode_commit_scaled`` when
    ``state_scale`` is given); accept: int32 [B] on the device, or None for
    all T drafts."""
    import torch
    if k.dim() != 4:
        raise ValueError("k must be [B, H, T, d]")
    B, H, T, d = k.shape
    _check(v, "v", (B, H, T, d), k.dtype, k.device)
    _check(state, "state", (B, H, d, d), None, k.device)
    if accept is not None:
        _check(accept, "accept", (B,), torch.int32, k.device)
    acc_ptr = accept.data_ptr() if accept is not None else None
    if state_scale is None:
        rc = library().lin_attn_decode_commit(k.data_ptr(), v.data_ptr(), state.data_ptr(), acc_ptr,
                                              B, H, T, d, _dtype_code(k), _dtype_code(state),
                                              _stream(stream, k.device))
        where = "lin_attn_decode_commit"
    else:
        rc = library().lin_attn_decode_commit_scaled(k.data_ptr(), v.data_ptr(), state.data_ptr(),
                                                     _scale_ptr(state_scale, B, H, k.device), acc_ptr,
                                                     B, H, T, d, _dtype_code(k), _dtype_code(state),
                                                     _stream(stream, k.device))
        where = "lin_attn_decode_commit_scaled"
    if rc != OK:
        raise LinAttnError(rc, where)
    return state


# how the dV and dK passes run (lin_attn_backward_ex)
BWD_AUTO, BWD_SEPARATE, BWD_PAIRED, BWD_FUSED = 0, 1, 2, 3


def backward(q, k, v, dout, dq, dk, dv, block: int, *, state0=None, dstate=None, dstate0=None, strategy=BWD_AUTO,
             stream=None):
    """Gradients of the chunked prefill (``lin_attn_backward``).

    q, k, v, dout, dq, dk, dv: [B, H, N, d] bf16 or fp32, one dtype (dq, dk,
    dv written);
    state0 (the forward call's S_0), dstate (gradient of the final state)
    and dstate0 (written: gradient of S_0): [B, H, d, d] fp32 or None."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, (B, H, N, d), q.dtype, q.device)
    ptrs = []
    for name, t in (("state0", state0), ("dstate", dstate), ("dstate0", dstate0)):
        if t is None:
            ptrs.append(None)
        else:
            _check(t, name, (B, H, d, d), torch.float32, q.device)
            ptrs.append(t.data_ptr())
    rc = library().lin_attn_backward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), ptrs[0],
                                        ptrs[1], dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ptrs[2], B, H, N, d,
                                        int(block), _dtype_code(q), int(strategy), _stream(stream, q.device))
    if rc != OK:
        raise LinAttnError(rc, "lin_attn_backward_ex")
    return dq, dk, dv
