"""C-ABI contract checks that need no GPU.

The library must load, export every function that include/lin_attn.h
declares, and reject bad arguments on the host before any HIP call (so these
calls are safe on a machine without a device).  No call here passes
validation with work to do, so no kernel is ever launched.  The module runs
only in a child process that sees no device (HIP_VISIBLE_DEVICES=-1, started
by test_abi_no_device.py): should a check ever pass by mistake, the launch
then fails with LIN_ATTN_EHIP instead of reaching a GPU with the fake
pointers these tests pass.
"""
import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_lightning_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lin_attn.h")

pytestmark = pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") != "-1",
                                reason="runs in a child process without a visible device (test_abi_no_device.py)")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails or returns first
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lin_attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("lin_attn_prefill", "lin_attn_prefill_ex", "lin_attn_decode", "lin_attn_decode_scaled",
              "lin_attn_prefill_scaled", "lin_attn_prefill_recurrent", "lin_attn_state_accumulate",
              "lin_attn_backward",
              "lin_attn_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = la.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in nm.stdout.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name


def test_library_is_gfx950_only(tmp_path):
    """The device code bundled into the library targets gfx950 and nothing else."""
    fb = tmp_path / "fatbin.bin"
    # objcopy rewrites its input unless an output file is named; name a scratch copy
    subprocess.run(["objcopy", f"--dump-section=.hip_fatbin={fb}", la.LIB_PATH, str(tmp_path / "scratch.so")],
                   check=True)
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          f"--input={fb}"], capture_output=True, text=True, check=True)
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets and all(t.endswith("gfx950") for t in targets), out.stdout


def test_strerror():
    assert la.strerror(la.OK) == "success"
    for c in (la.EINVAL, la.EUNSUPPORTED, la.EHIP, la.ESCRATCH):
        assert la.strerror(c) and la.strerror(c) != "success"
    assert "unknown" in la.strerror(12345)


def prefill(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, s=FAKE, B=1, H=1, N=16, d=128, block=64, dt=la.BF16, split=0):
    return lib.lin_attn_prefill_ex(q, k, v, o, s, B, H, N, d, block, dt, split, None)


def test_prefill_validation_codes():
    lib = la.library()
    # negative sizes
    for kw in ({"B": -1}, {"H": -1}, {"N": -1}, {"d": -1}, {"block": -1}, {"split": -1}):
        assert prefill(lib, **kw) == la.EINVAL, kw
    # unsupported head dims, block sizes, dtypes and splits
    for kw in ({"d": 32}, {"d": 96}, {"d": 256}, {"block": 0}, {"block": 8}, {"block": 40},
               {"block": 144}, {"d": 128, "block": 256}, {"dt": 7}, {"split": 3}, {"split": 8},
               {"d": 64, "block": 64, "split": 4}, {"dt": la.F32, "block": 128},
               {"dt": la.F32, "split": 2}):
        assert prefill(lib, **kw) == la.EUNSUPPORTED, kw
    # zero work is a successful no-op, even with null pointers
    for kw in ({"B": 0}, {"H": 0}, {"N": 0}):
        assert prefill(lib, q=None, k=None, v=None, o=None, s=None, **kw) == la.OK, kw
    # null or misaligned pointers with work to do
    for name in ("q", "k", "v", "o", "s"):
        assert prefill(lib, **{name: None}) == la.EINVAL, name
        assert prefill(lib, **{name: MISALIGNED}) == la.EINVAL, name
    # size products that overflow int64
    assert prefill(lib, B=1 << 40, H=1 << 30) == la.EINVAL


def test_prefill_plain_entry_matches_ex_validation():
    lib = la.library()
    assert lib.lin_attn_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 100, 64, la.BF16, None) == la.EUNSUPPORTED
    assert lib.lin_attn_prefill(None, None, None, None, None, 1, 1, 0, 128, 64, la.BF16, None) == la.OK
    assert lib.lin_attn_prefill(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 128, 64, la.BF16, None) == la.EINVAL


def test_supported_block_sizes_are_accepted_by_validation():
    """Every supported block passes the size checks: with a null q the call then
    fails on the pointer check (EINVAL), never on the block (EUNSUPPORTED)."""
    lib = la.library()
    for d, maxblk in ((128, 128), (64, 128)):
        for block in range(16, maxblk + 1, 16):
            assert prefill(lib, q=None, d=d, block=block) == la.EINVAL, (d, block)
        assert prefill(lib, q=None, d=d, block=maxblk + 16) == la.EUNSUPPORTED, d
    for d, maxblk in ((128, 64), (64, 128)):
        for block in range(16, maxblk + 1, 16):
            assert prefill(lib, q=None, d=d, block=block, dt=la.F32) == la.EINVAL, (d, block)


def test_decode_validation_codes():
    lib = la.library()

    def dec(q=FAKE, k=FAKE, v=FAKE, o=FAKE, s=FAKE, B=1, H=1, d=128, io=la.BF16, st=la.F32):
        return lib.lin_attn_decode(q, k, v, o, s, B, H, d, io, st, None)

    assert dec(B=-1) == la.EINVAL
    assert dec(d=96) == la.EUNSUPPORTED
    assert dec(io=5) == la.EUNSUPPORTED
    assert dec(st=5) == la.EUNSUPPORTED
    assert dec(B=0, q=None, k=None, v=None, o=None, s=None) == la.OK
    for name in ("q", "k", "v", "o", "s"):
        assert dec(**{name: None}) == la.EINVAL
        assert dec(**{name: MISALIGNED}) == la.EINVAL


def test_scaled_state_validation_codes():
    lib = la.library()
    SC = FAKE  # any aligned non-null address: never dereferenced by a rejected call

    def dec(q=FAKE, s=FAKE, sc=SC, B=1, H=1, d=128, io=la.BF16, st=la.FP8_E4M3):
        return lib.lin_attn_decode_scaled(q, FAKE, FAKE, FAKE, s, sc, B, H, d, io, st, None)

    assert dec(B=-1) == la.EINVAL
    assert dec(st=la.F32) == la.EUNSUPPORTED  # fp32 states are not scaled
    assert dec(st=7) == la.EUNSUPPORTED
    assert dec(d=32) == la.EUNSUPPORTED
    assert dec(q=None) == la.EINVAL and dec(s=MISALIGNED) == la.EINVAL
    assert dec(sc=FAKE + 2) == la.EINVAL  # scales are float-aligned
    assert dec(B=0, q=None, s=None, sc=None) == la.OK
    # the plain entry point takes an FP8 state too (unit scales)
    assert lib.lin_attn_decode(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, la.BF16, la.FP8_E4M3, None) == la.EINVAL
    assert lib.lin_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 96, la.BF16, la.FP8_E4M3, None) == la.EUNSUPPORTED

    def pre(q=FAKE, s=FAKE, sc=SC, B=1, H=1, N=16, d=128, block=64, io=la.BF16, st=la.BF16, rc=0):
        return lib.lin_attn_prefill_scaled(q, FAKE, FAKE, FAKE, s, sc, B, H, N, d, block, io, st, rc, None)

    for kw in ({"B": -1}, {"N": -1}, {"rc": 2}, {"rc": -1}, {"q": None}, {"s": None}, {"s": MISALIGNED},
               {"sc": FAKE + 1}):
        assert pre(**kw) == la.EINVAL, kw
    for kw in ({"st": la.F32}, {"st": 9}, {"io": la.F32}, {"d": 96}, {"block": 144}, {"block": 40}):
        assert pre(**kw) == la.EUNSUPPORTED, kw
    for st in (la.BF16, la.FP8_E4M3):
        for rc in (0, 1):
            assert pre(N=0, q=None, s=None, sc=None, st=st, rc=rc) == la.OK
            assert pre(q=None, st=st, rc=rc, sc=None) == la.EINVAL  # passes every size check


def test_scaled_verify_commit_validation_codes():
    lib = la.library()

    def ver(q=FAKE, s=FAKE, sc=None, B=1, H=1, T=4, d=128, io=la.BF16, st=la.FP8_E4M3):
        return lib.lin_attn_decode_verify_scaled(q, FAKE, FAKE, FAKE, s, sc, B, H, T, d, io, st, None)

    def com(s=FAKE, sc=None, acc=None, B=1, H=1, T=4, d=128, io=la.BF16, st=la.FP8_E4M3):
        return lib.lin_attn_decode_commit_scaled(FAKE, FAKE, s, sc, acc, B, H, T, d, io, st, None)

    for f in (ver, com):
        assert f(st=la.F32) == la.EUNSUPPORTED
        assert f(st=7) == la.EUNSUPPORTED
        assert f(T=17) == la.EUNSUPPORTED
        assert f(B=-1) == la.EINVAL
        assert f(s=None) == la.EINVAL
        assert f(sc=FAKE + 2) == la.EINVAL
        assert f(T=0, s=None) == la.OK
    assert ver(q=None) == la.EINVAL
    assert com(acc=FAKE + 1) == la.EINVAL
    # the unscaled calls accept an FP8 state (unit scales)
    assert lib.lin_attn_decode_verify(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 4, 128, la.BF16, la.FP8_E4M3, None) == la.EINVAL
    assert lib.lin_attn_decode_commit(FAKE, FAKE, FAKE, None, 1, 1, 4, 96, la.BF16, la.FP8_E4M3, None) == la.EUNSUPPORTED


def test_backward_validation_codes():
    lib = la.library()

    def bwd(q=FAKE, dq=FAKE, s0=None, ds=None, ds0=None, B=1, H=1, N=16, d=128, block=64, io=la.BF16):
        return lib.lin_attn_backward(q, FAKE, FAKE, FAKE, s0, ds, dq, FAKE, FAKE, ds0, B, H, N, d, block, io, None)

    for kw in ({"B": -1}, {"N": -1}, {"block": -1}, {"q": None}, {"dq": None}, {"q": MISALIGNED},
               {"s0": MISALIGNED}, {"ds": MISALIGNED}, {"ds0": MISALIGNED}, {"B": 1 << 40, "H": 1 << 30}):
        assert bwd(**kw) == la.EINVAL, kw
    for kw in ({"io": 9}, {"d": 96}, {"block": 144}, {"block": 8}, {"block": 40},
               {"io": la.F32, "block": 128}):  # fp32 I/O: blocks up to 64 at d = 128
        assert bwd(**kw) == la.EUNSUPPORTED, kw
    assert bwd(B=0, q=None, dq=None) == la.OK
    assert bwd(N=0, q=None, dq=None) == la.OK  # no tokens and no dS_0 requested: nothing to do


def test_recurrent_validation_codes():
    lib = la.library()

    def rec(q=FAKE, B=1, H=1, N=8, d=128, io=la.BF16):
        return lib.lin_attn_prefill_recurrent(q, FAKE, FAKE, FAKE, FAKE, B, H, N, d, io, None)

    assert rec(N=-1) == la.EINVAL
    assert rec(d=48) == la.EUNSUPPORTED
    assert rec(io=3) == la.EUNSUPPORTED
    assert rec(N=0, q=None) == la.OK
    assert rec(q=None) == la.EINVAL
    assert rec(q=MISALIGNED) == la.EINVAL


def test_binding_rejects_bad_tensors_without_a_device():
    import torch
    x = torch.zeros(1, 1, 16, 128, dtype=torch.bfloat16)  # CPU tensor
    s = torch.zeros(1, 1, 128, 128)
    with pytest.raises(ValueError):
        la.prefill(x, x, x, x, s, 64)
    with pytest.raises(ValueError):
        la.decode(x[:, :, 0], x[:, :, 0], x[:, :, 0], x[:, :, 0], s)


def test_state_accumulate_validation_codes():
    lib = la.library()

    def acc(k=FAKE, v=FAKE, s=FAKE, B=1, H=1, N=8, d=128, io=la.BF16):
        return lib.lin_attn_state_accumulate(k, v, s, B, H, N, d, io, None)

    for kw in ({"B": -1}, {"H": -1}, {"N": -1}, {"d": -1}):
        assert acc(**kw) == la.EINVAL, kw
    for kw in ({"d": 32}, {"d": 96}, {"io": 4}):
        assert acc(**kw) == la.EUNSUPPORTED, kw
    for kw in ({"B": 0}, {"H": 0}, {"N": 0}):
        assert acc(k=None, v=None, s=None, **kw) == la.OK, kw
    for name in ("k", "v", "s"):
        assert acc(**{name: None}) == la.EINVAL, name
        assert acc(**{name: MISALIGNED}) == la.EINVAL, name
    assert acc(B=1 << 40, H=1 << 30) == la.EINVAL


def test_snapshot_validation_codes():
    lib = la.library()

    def snp(snap=FAKE, N=256, block=64, every=1, q=FAKE, d=128):
        return lib.lin_attn_prefill_snapshots(q, FAKE, FAKE, FAKE, FAKE, snap, 1, 1, N, d, block, every,
                                              la.BF16, None)

    assert snp(every=0) == la.EINVAL
    assert snp(every=-3) == la.EINVAL
    assert snp(block=40) == la.EUNSUPPORTED
    assert snp(snap=None) == la.EINVAL          # 4 snapshots due, no buffer
    assert snp(snap=MISALIGNED) == la.EINVAL
    assert snp(q=None) == la.EINVAL
    assert snp(N=0, q=None, snap=None) == la.OK


def test_decode_multi_validation_codes():
    lib = la.library()

    def ver(q=FAKE, o=FAKE, s=FAKE, B=1, H=1, T=4, d=128, io=la.BF16, st=la.F32):
        return lib.lin_attn_decode_verify(q, FAKE, FAKE, o, s, B, H, T, d, io, st, None)

    def com(k=FAKE, s=FAKE, acc=None, B=1, H=1, T=4, d=128, io=la.BF16, st=la.F32):
        return lib.lin_attn_decode_commit(k, FAKE, s, acc, B, H, T, d, io, st, None)

    for f in (ver, com):
        assert f(T=-1) == la.EINVAL
        assert f(B=-1) == la.EINVAL
        assert f(T=17) == la.EUNSUPPORTED
        assert f(d=96) == la.EUNSUPPORTED
        assert f(io=3) == la.EUNSUPPORTED
        assert f(st=3) == la.EUNSUPPORTED
        assert f(T=0, s=None) == la.OK
        assert f(s=None) == la.EINVAL
        assert f(s=MISALIGNED) == la.EINVAL
    assert ver(q=None) == la.EINVAL
    assert ver(o=MISALIGNED) == la.EINVAL
    assert com(k=None) == la.EINVAL
    assert com(acc=FAKE + 2) == la.EINVAL   # accept must be 4-byte aligned


def test_stream_probe_is_a_separate_library():
    """The bandwidth probe that bench.py uses lives in its own library: it
    exports hbm_stream, rejects bad arguments on the host, and the attention
    library does not contain it."""
    probe = os.path.join(os.path.dirname(la.LIB_PATH), "libhbm_stream.so")
    lib = ctypes.CDLL(probe)
    lib.hbm_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.hbm_stream(None, FAKE, 1, 1, 1, 0, 1, 1, None) == -1
    assert lib.hbm_stream(FAKE, FAKE, -1, 1, 1, 0, 1, 1, None) == -1
    assert lib.hbm_stream(FAKE, FAKE, 0, 1, 1, 0, 1, 1, None) == 0  # nothing to do: no launch
    assert lib.hbm_stream(FAKE, FAKE, 1, 3, 1, 0, 1, 1, None) == -2  # in place needs one read per write
    assert lib.hbm_stream(FAKE, FAKE, 1, 1, 0, 0, 1, 1, None) == -2  # an in-place run must write
    assert lib.hbm_stream(FAKE, FAKE, 1, 1, 1, 0, 1, 2, None) == -2  # batch is 1, 4 or 16
    lib.hbm_stream_roles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p]
    assert lib.hbm_stream_roles(None, FAKE, 1, 0, 1, 8, None) == -1
    assert lib.hbm_stream_roles(FAKE, FAKE, 1, 0, 1, 8, None) == -1      # src and dst must differ
    assert lib.hbm_stream_roles(FAKE, FAKE + 16, 1, 0, 1, 5, None) == -2  # depth is 4, 8 or 16
    assert lib.hbm_stream_roles(FAKE, FAKE + 16, 0, 0, 1, 8, None) == 0   # nothing to do: no launch
    nm = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True, text=True, check=True)
    assert "hbm_stream" not in nm.stdout


def test_split_accumulation_workspace_query_and_validation():
    """The workspace query and the split accumulation reject what the call
    rejects, before any launch; too small a workspace is EINVAL.  A query
    with work to plan needs the device's compute-unit count: without a
    device it returns LIN_ATTN_EHIP (the sizes are checked on the GPU)."""
    lib = la.library()
    q = lib.lin_attn_state_accumulate_split_workspace
    assert q(1, 64, 131072, 128, la.BF16) == la.EHIP  # plan needs the device
    assert q(1, 2, 3000, 64, la.F32) == 0             # fp32 I/O: the unsplit kernel
    assert q(1, 2, 0, 128, la.BF16) == 0              # nothing to do
    assert q(1, 2, 100, 96, la.BF16) == la.EUNSUPPORTED
    assert q(-1, 2, 100, 64, la.BF16) == la.EINVAL
    assert q(1, 2, 100, 64, 7) == la.EUNSUPPORTED
    f = lib.lin_attn_state_accumulate_split
    assert f(FAKE, FAKE, FAKE, 1, 8, 4096, 96, la.BF16, FAKE, 1 << 20, None) == la.EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 1, -8, 4096, 128, la.BF16, FAKE, 1 << 20, None) == la.EINVAL
    assert f(FAKE, FAKE, FAKE, 1, 8, 4096, 128, la.BF16, FAKE, 1 << 20, None) == la.EHIP  # no device
    assert f(FAKE, FAKE, FAKE, 1, 8, 0, 128, la.BF16, None, 0, None) == la.OK  # nothing to do


def test_seqsplit_workspace_query_and_validation():
    lib = la.library()
    q = lib.lin_attn_prefill_seqsplit_workspace
    assert q(1, 64, 131072, 128, 128, la.BF16) == la.EHIP  # plan needs the device
    assert q(1, 8, 4096, 128, 64, la.F32) == 0          # fp32 I/O: the uncut prefill
    assert q(1, 8, 0, 128, 128, la.BF16) == 0           # nothing to do
    assert q(1, 8, 4096, 128, 100, la.BF16) == la.EUNSUPPORTED
    assert q(1, 8, 4096, 96, 128, la.BF16) == la.EUNSUPPORTED
    assert q(1, -8, 4096, 128, 128, la.BF16) == la.EINVAL
    f = lib.lin_attn_prefill_seqsplit
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8192, 128, 128, la.BF16)
    assert f(*args, FAKE, 1 << 30, None) == la.EHIP       # no device to plan on
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8192, 96, 128, la.BF16, FAKE, 1 << 30, None) == la.EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8192, 128, 100, la.BF16, FAKE, 1 << 30, None) == la.EUNSUPPORTED


def test_seqsplit_noalloc_validation():
    """The scratch-buffer variant rejects what the workspace variant rejects,
    and reports its fixed buffer size; it needs no workspace arguments."""
    lib = la.library()
    assert lib.lin_attn_scratch_bytes() == 56 << 20
    f = lib.lin_attn_prefill_seqsplit_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8192, 96, 128, la.BF16, None) == la.EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8192, 128, 100, la.BF16, None) == la.EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 8192, 128, 128, la.BF16, None) == la.EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8192, 128, 128, 7, None) == la.EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 0, 128, 128, la.BF16, None) == la.OK  # nothing to do
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 8192, 128, 128, la.BF16, None) == la.EHIP  # no device


def test_backward_strategy_validation():
    lib = la.library()
    f = lib.lin_attn_backward_ex
    args = (FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, 1, 2, 100, 128, 128, la.BF16)
    assert f(*args, 4, None) == la.EINVAL
    assert f(*args, -1, None) == la.EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, 1, 2, 100, 96, 128, la.BF16, 3, None) \
        == la.EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, 0, 2, 100, 128, 128, la.BF16, 3, None) \
        == la.OK  # no sequences: nothing to do
