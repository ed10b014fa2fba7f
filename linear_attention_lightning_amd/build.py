"""Build the gfx950 shared library ``_lib/liblin_attn.so`` in place.

Usage: ``python -m linear_attention_lightning_amd.build`` (or ``build()``).
Every HIP source is compiled by hipcc for gfx950 only; the objects are linked
into one shared library that exports the C ABI of include/lin_attn.h.  A
second, separate library ``_lib/libhbm_stream.so`` holds the streaming
bandwidth probe that bench.py measures the HBM ceiling of a traffic mix with
(csrc/hbm_stream.h); the attention library does not contain it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "liblin_attn.so")
PROBE_LIB = os.path.join(OUT_DIR, "libhbm_stream.so")
PROBE_SOURCES = ["hbm_stream.hip"]
SOURCES = ["lin_attn_api.hip", "prefill_bf16.hip", "prefill_bf16_scaled.hip", "prefill_bf16_grad.hip", "prefill_f32.hip", "decode.hip", "recurrent.hip",
           "state_delta.hip", "decode_multi.hip"]

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed-fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    for line in res.stderr.splitlines():
        if "packed-fp32-ops" in line and "not a recognized feature" in line:
            continue  # the host pass does not know the device feature; harmless
        if line.strip():
            print(line, file=sys.stderr)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, min(os.cpu_count() or 1, 8)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, obj_dir), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
