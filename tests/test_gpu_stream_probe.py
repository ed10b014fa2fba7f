"""The streaming probe behind the HBM ceilings (libhbm_stream.so) writes what
it is asked to write, for every mix, store policy and batch depth, over a
ragged split of units across workgroups.  A probe that skipped work would
report a ceiling no kernel could reach; these checks pin the values it moves
(bench.py additionally rejects any rate above the HBM peak)."""
import ctypes
import itertools
import os

import pytest
import torch

import linear_attention_lightning_amd as la

from gpu_helpers import announce

pytestmark = pytest.mark.gpu

UNIT = 4096            # bytes per slice
UNITS = 1000           # not a multiple of any batch times the grid below
WORKGROUPS = 7         # 143 units per workgroup, 142 for the last


def probe():
    lib = ctypes.CDLL(os.path.join(os.path.dirname(la.LIB_PATH), "libhbm_stream.so"))
    lib.hbm_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def run(lib, src, dst, rd, write, nt, batch):
    stream = torch.cuda.current_stream()
    assert src.numel() * 4 >= UNITS * rd * UNIT and dst.numel() * 4 >= (UNITS if write else 1) * UNIT
    rc = lib.hbm_stream(src.data_ptr(), dst.data_ptr(), UNITS, rd, write, nt, WORKGROUPS, batch, stream.cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0


@pytest.mark.parametrize("rd,nt,batch", list(itertools.product((1, 3), (0, 1), (1, 4, 16))))
def test_stream_writes_the_xor_of_its_slices(rd, nt, batch):
    announce("stream probe", rd, nt, batch)
    lib = probe()
    g = torch.Generator(device="cuda").manual_seed(100 + 10 * rd + batch)
    src = torch.randint(-2**31, 2**31 - 1, (UNITS * rd * UNIT // 4,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.full((UNITS * UNIT // 4,), 7, dtype=torch.int32, device="cuda")
    run(lib, src, dst, rd, 1, nt, batch)
    slices = src.view(UNITS, rd, UNIT // 4)
    want = slices[:, 0]
    for r in range(1, rd):
        want = want ^ slices[:, r]
    assert torch.equal(dst.view(UNITS, UNIT // 4), want)


@pytest.mark.parametrize("nt,batch", list(itertools.product((0, 1), (1, 4, 16))))
def test_in_place_stream_leaves_the_buffer_as_it_was(nt, batch):
    announce("stream probe in place", nt, batch)
    lib = probe()
    g = torch.Generator(device="cuda").manual_seed(200 + batch)
    buf = torch.randint(-2**31, 2**31 - 1, (UNITS * UNIT // 4,), dtype=torch.int32, device="cuda", generator=g)
    before = buf.clone()
    run(lib, buf, buf, 1, 1, nt, batch)
    assert torch.equal(buf, before)


@pytest.mark.parametrize("batch", (1, 4, 16))
def test_read_only_stream_stores_nothing_for_equal_bytes(batch):
    announce("stream probe read only", batch)
    lib = probe()
    src = torch.ones((UNITS * UNIT // 4,), dtype=torch.int32, device="cuda")
    dst = torch.full((2 * UNIT // 4,), 7, dtype=torch.int32, device="cuda")
    run(lib, src, dst, 1, 0, 0, batch)
    # equal bytes everywhere: the guarded store never happens
    assert torch.all(dst == 7)


@pytest.mark.parametrize("nt,depth", list(itertools.product((0, 1), (4, 8, 16))))
def test_role_split_stream_writes_its_pattern_and_reads_everything(nt, depth):
    """The role-split reference (three reading waves, one writing wave per
    workgroup) fills every written unit with its pattern, and its reads of
    equal bytes never take the guarded store."""
    announce("stream probe roles", nt, depth)
    lib = probe()
    lib.hbm_stream_roles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p]
    src = torch.ones((3 * UNITS * UNIT // 4,), dtype=torch.int32, device="cuda")
    dst = torch.full((UNITS * UNIT // 4,), 7, dtype=torch.int32, device="cuda")
    rc = lib.hbm_stream_roles(src.data_ptr(), dst.data_ptr(), UNITS, nt, WORKGROUPS, depth,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    pattern = torch.tensor([0x9e3779b9, 0x7f4a7c15, 0x94d049bb, 0x2545f491], dtype=torch.int64).to(torch.int32)
    assert torch.equal(dst.view(-1, 4).cpu(), pattern.expand(UNITS * UNIT // 16, 4))
